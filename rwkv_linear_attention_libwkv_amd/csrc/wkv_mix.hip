// Token shift of the time-mixing block for gfx950.
//
// Page "Reinventing RNNs for the Transformer Era: RWKV" (velog review), section "토큰 변환":
// the block forms the inputs of its R, K, V projections by linear interpolation between the
// current and the previous time step.  For M mix vectors mu_m (per channel):
//   out_m[b, t, c] = mu_m[c] x[b, t, c] + (1 - mu_m[c]) x[b, t-1, c],
// with x[b, -1, c] the token before the sequence (x_prev, or zero).  Computed as
// fma(mu, x_t, (1 - mu) x_{t-1}): within two roundings of |mu x_t| + |(1 - mu) x_{t-1}|
// (the form mu (x_t - x_{t-1}) + x_{t-1} loses that bound when x_{t-1} dominates and mu ~ 1).
//
// Elementwise and HBM-bound: a thread owns a 16-byte vector of channels (4 float32 or 8
// bfloat16) over a segment of kShiftSeg time steps, so each x element is read once (plus one
// row per segment for x_{t-1}) and the M outputs are written once; consecutive threads take
// consecutive vectors of a row, so every wave access is one contiguous 1 KB segment.  Rows
// of a C that is not a multiple of the vector (or unaligned arrays) take one element per
// thread.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wkv_kernels.h"
#include "wkv_rows.h"

namespace wkv {

constexpr int kShiftSeg = 32;

template <typename IO, int VEC>
struct Vec;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <>
struct Vec<float, 4> {
    typedef f32x4 raw;
    static __device__ __forceinline__ void to_f(const raw& r, float (&f)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = r[i];
    }
    static __device__ __forceinline__ raw from_f(const float (&f)[4]) { return raw{f[0], f[1], f[2], f[3]}; }
};
template <>
struct Vec<uint16_t, 8> {
    typedef u32x4 raw;
    static __device__ __forceinline__ void to_f(const raw& r, float (&f)[8]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = bf_lo(r[i]);
            f[2 * i + 1] = bf_hi(r[i]);
        }
    }
    static __device__ __forceinline__ raw from_f(const float (&f)[8]) {
        return raw{pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]), pack_bf16(f[4], f[5]), pack_bf16(f[6], f[7])};
    }
};
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <>
struct Vec<uint16_t, 4> {
    typedef u32x2 raw;
    static __device__ __forceinline__ void to_f(const raw& r, float (&f)[4]) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            f[2 * i] = bf_lo(r[i]);
            f[2 * i + 1] = bf_hi(r[i]);
        }
    }
    static __device__ __forceinline__ raw from_f(const float (&f)[4]) {
        return raw{pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3])};
    }
};
template <typename IO>
struct Vec<IO, 1> {
    typedef IO raw;
    static __device__ __forceinline__ void to_f(const raw& r, float (&f)[1]) {
        if constexpr (sizeof(IO) == 4)
            f[0] = r;
        else
            f[0] = bf_lo((uint32_t)r);
    }
    static __device__ __forceinline__ raw from_f(const float (&f)[1]) {
        if constexpr (sizeof(IO) == 4)
            return f[0];
        else
            return (IO)(pack_bf16(f[0], 0.f) & 0xffffu);
    }
};

template <typename IO, int VEC>
__global__ __launch_bounds__(256) void token_shift_kernel(ShiftArgs a) {
    typedef Vec<IO, VEC> V;
    typedef typename V::raw raw;
    const long nv = a.C / VEC;  // vectors per row
    const long n_seg = (a.T + kShiftSeg - 1) / kShiftSeg;
    const long tid = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (tid >= (long)a.B * n_seg * nv) return;
    const long cv = tid % nv;
    const long seg = (tid / nv) % n_seg;
    const long b = tid / (nv * n_seg);
    const long c0 = cv * VEC;

    float mu[kShiftMaxM][VEC];
#pragma unroll
    for (int m = 0; m < kShiftMaxM; ++m)
#pragma unroll
        for (int i = 0; i < VEC; ++i) mu[m][i] = m < a.M ? a.mu[(long)m * a.C + c0 + i] : 0.f;

    const raw* x = static_cast<const raw*>(a.x) + (b * a.T) * nv + cv;
    const long t0 = seg * kShiftSeg;
    const int n = (int)min((long)kShiftSeg, (long)a.T - t0);
    float prev[VEC];
    if (t0 > 0) {
        V::to_f(__builtin_nontemporal_load(x + (t0 - 1) * nv), prev);
    } else if (a.x_prev) {
        V::to_f(static_cast<const raw*>(a.x_prev)[b * nv + cv], prev);
    } else {
#pragma unroll
        for (int i = 0; i < VEC; ++i) prev[i] = 0.f;
    }
    const long plane = (long)a.B * a.T * nv;  // vectors per output
    raw* out = static_cast<raw*>(a.out) + (b * a.T) * nv + cv;
#pragma unroll 4
    for (int j = 0; j < n; ++j) {
        const long t = t0 + j;
        float cur[VEC];
        V::to_f(__builtin_nontemporal_load(x + t * nv), cur);
#pragma unroll
        for (int m = 0; m < kShiftMaxM; ++m) {
            if (m >= a.M) break;
            float o[VEC];
#pragma unroll
            for (int i = 0; i < VEC; ++i) o[i] = fmaf(mu[m][i], cur[i], (1.f - mu[m][i]) * prev[i]);
            __builtin_nontemporal_store(V::from_f(o), out + m * plane + t * nv);
        }
#pragma unroll
        for (int i = 0; i < VEC; ++i) prev[i] = cur[i];
    }
}

// Backward of the token shift: for L = sum_m sum g_m * out_m,
//   dL/dx_t      = sum_m mu_m g_{m,t} + (1 - mu_m) g_{m,t+1}    (g_{m,T} = 0)
//   dL/dmu_m     = sum_t g_{m,t} (x_t - x_{t-1})                 (per (b, c) lane)
//   dL/dx_prev   = sum_m (1 - mu_m) g_{m,0}.
// A thread owns a vector of channels (4, or 8 bf16 channels, see launch_token_shift_backward)
// over kShiftSeg steps; each
// thread writes dL/dx of its segment and its segment's partial sums of dL/dmu, which
// token_shift_reduce_kernel adds per lane in a fixed order in float64 (deterministic, and the
// sum over T keeps float32 partials of kShiftSeg terms only).
template <typename IO, int VEC, int M>
__global__ __launch_bounds__(256) void token_shift_bwd_kernel(ShiftBwdArgs a) {
    typedef Vec<IO, VEC> V;
    typedef typename V::raw raw;
    const long nv = a.C / VEC;
    const long n_seg = (a.T + kShiftSeg - 1) / kShiftSeg;
    const long tid = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (tid >= (long)a.B * n_seg * nv) return;
    const long cv = tid % nv;
    const long seg = (tid / nv) % n_seg;
    const long b = tid / (nv * n_seg);
    const long c0 = cv * VEC;

    float mu[M][VEC];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int i = 0; i < VEC; ++i) mu[m][i] = a.mu[(long)m * a.C + c0 + i];

    const raw* x = static_cast<const raw*>(a.x) + (b * a.T) * nv + cv;
    const raw* g = static_cast<const raw*>(a.g) + (b * a.T) * nv + cv;
    raw* gx = static_cast<raw*>(a.gx) + (b * a.T) * nv + cv;
    const long plane = (long)a.B * a.T * nv;  // vectors per mix of g
    const long t0 = seg * kShiftSeg;
    const int n = (int)min((long)kShiftSeg, (long)a.T - t0);
    float prev[VEC];
    if (t0 > 0) {
        V::to_f(__builtin_nontemporal_load(x + (t0 - 1) * nv), prev);
    } else if (a.x_prev) {
        V::to_f(static_cast<const raw*>(a.x_prev)[b * nv + cv], prev);
    } else {
#pragma unroll
        for (int i = 0; i < VEC; ++i) prev[i] = 0.f;
    }
    float gmu[M][VEC];
    float gcur[M][VEC];  // g_{m,t}
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
            gmu[m][i] = 0.f;
            gcur[m][i] = 0.f;
        }
#pragma unroll
    for (int m = 0; m < M; ++m)
        V::to_f(__builtin_nontemporal_load(g + m * plane + t0 * nv), gcur[m]);
    if (seg == 0 && a.gprev) {  // dL/dx_prev = sum_m (1 - mu_m) g_{m,0}
        float gp[VEC];
#pragma unroll
        for (int i = 0; i < VEC; ++i) gp[i] = 0.f;
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int i = 0; i < VEC; ++i) gp[i] = fmaf(1.f - mu[m][i], gcur[m][i], gp[i]);
        static_cast<raw*>(a.gprev)[b * nv + cv] = V::from_f(gp);
    }
    // two steps per round, so that the loads of both are in flight together (a bf16 step of 4
    // channels reads only 8 bytes per lane and array: one step at a time leaves the loads
    // latency-bound); 8 bf16 channels (16-byte vectors) take one step per round, whose loads
    // already move as many bytes, since two would cost a wave per SIMD in registers
    constexpr int kStepsPerRound = (sizeof(IO) == 2 && VEC == 8) ? 1 : 2;
#pragma unroll kStepsPerRound
    for (int j = 0; j < n; ++j) {
        const long t = t0 + j;
        float cur[VEC], d[VEC], o[VEC];
        V::to_f(__builtin_nontemporal_load(x + t * nv), cur);
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
            d[i] = cur[i] - prev[i];
            o[i] = 0.f;
            prev[i] = cur[i];
        }
        const bool last = t + 1 >= a.T;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            float gn[VEC];
            if (last) {
#pragma unroll
                for (int i = 0; i < VEC; ++i) gn[i] = 0.f;
            } else {
                V::to_f(__builtin_nontemporal_load(g + m * plane + (t + 1) * nv), gn);
            }
#pragma unroll
            for (int i = 0; i < VEC; ++i) {
                o[i] = fmaf(mu[m][i], gcur[m][i], fmaf(1.f - mu[m][i], gn[i], o[i]));
                gmu[m][i] = fmaf(gcur[m][i], d[i], gmu[m][i]);
                gcur[m][i] = gn[i];
            }
        }
        __builtin_nontemporal_store(V::from_f(o), gx + t * nv);
    }
    // partial sums: part[seg][m][b][c]
#pragma unroll
    for (int m = 0; m < M; ++m) {
        float* dst = a.part + ((seg * a.M + m) * a.B + b) * (long)a.C + c0;
#pragma unroll
        for (int i = 0; i < VEC; ++i) dst[i] = gmu[m][i];
    }
}

// dL/dmu per (m, b, c) lane: the segments' partial sums added in float64, in a fixed order.
// Block: 64 lanes x kShiftRedSlices slices; slice k adds, in segment order, the k-th of
// kShiftRedSlices consecutive ranges of segments (loads unrolled by eight, so they are in
// flight together; a long sequence has thousands of segments per lane), and slice 0 then adds
// the slices' sums in slice order.
constexpr int kShiftRedSlices = 8;

__global__ __launch_bounds__(64 * kShiftRedSlices) void token_shift_reduce_kernel(ShiftBwdArgs a) {
    __shared__ double sums[kShiftRedSlices][64];
    const int lane = threadIdx.x & 63, slice = threadIdx.x >> 6;
    const long lanes = (long)a.M * a.B * a.C;
    const long i = (long)blockIdx.x * 64 + lane;
    const long n_seg = (a.T + kShiftSeg - 1) / kShiftSeg;
    const long per = (n_seg + kShiftRedSlices - 1) / kShiftRedSlices;
    const long s0 = slice * per, s1 = min(n_seg, s0 + per);
    double s = 0.0;
    if (i < lanes) {
#pragma unroll 8
        for (long seg = s0; seg < s1; ++seg) s += (double)a.part[seg * lanes + i];
    }
    sums[slice][lane] = s;
    __syncthreads();
    if (slice == 0 && i < lanes) {
        double t = 0.0;
#pragma unroll
        for (int k = 0; k < kShiftRedSlices; ++k) t += sums[k][lane];
        a.gmu[i] = (float)t;
    }
}

template <typename IO, int VEC>
static hipError_t launch_shift_bwd_t(const ShiftBwdArgs& a, hipStream_t s) {
    const long n_seg = (a.T + kShiftSeg - 1) / kShiftSeg;
    const long threads = (long)a.B * n_seg * (a.C / VEC);
    const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
    switch (a.M) {  // the number of mixes sizes the per-thread arrays
        case 1: hipLaunchKernelGGL((token_shift_bwd_kernel<IO, VEC, 1>), grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL((token_shift_bwd_kernel<IO, VEC, 2>), grid, block, 0, s, a); break;
        case 3: hipLaunchKernelGGL((token_shift_bwd_kernel<IO, VEC, 3>), grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL((token_shift_bwd_kernel<IO, VEC, 4>), grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    const long lanes = (long)a.M * a.B * a.C;
    hipLaunchKernelGGL(token_shift_reduce_kernel, dim3((unsigned)((lanes + 63) / 64)), dim3(64 * kShiftRedSlices), 0,
                       s, a);
    return hipGetLastError();
}

// vec: channels per thread, 8 (bf16 only: 16-byte vectors), 4 (16-byte float32 or 8-byte bf16
// vectors) or 1; C a multiple of it and x, x_prev, g, gx, gprev aligned to the vector.  With
// three bf16 mixes (B=1, T=65536, C=5120), 16-byte vectors: 687.1 against 769.9 us (four mixes
// 1007.9 against 1179.0); with one mix, 408.4 against 398.7, so one mix keeps 8-byte vectors.
hipError_t launch_token_shift_backward(const ShiftBwdArgs& a, int dtype, int vec, hipStream_t s) {
    if (dtype == 0) return vec >= 4 ? launch_shift_bwd_t<float, 4>(a, s) : launch_shift_bwd_t<float, 1>(a, s);
    if (vec == 8) return launch_shift_bwd_t<uint16_t, 8>(a, s);
    return vec == 4 ? launch_shift_bwd_t<uint16_t, 4>(a, s) : launch_shift_bwd_t<uint16_t, 1>(a, s);
}

long token_shift_segments(long T) { return (T + kShiftSeg - 1) / kShiftSeg; }

__global__ void zero_u16_kernel(uint16_t* __restrict__ p, long n) {
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) p[i] = 0;
}

hipError_t launch_zero_u16(void* p, long n, hipStream_t s) {
    const long blocks = n / 256 + 1 < 4096 ? n / 256 + 1 : 4096;
    hipLaunchKernelGGL(zero_u16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<uint16_t*>(p), n);
    return hipGetLastError();
}

template <typename IO, int VEC>
static hipError_t launch_shift_t(const ShiftArgs& a, hipStream_t s) {
    const long n_seg = (a.T + kShiftSeg - 1) / kShiftSeg;
    const long threads = (long)a.B * n_seg * (a.C / VEC);
    hipLaunchKernelGGL((token_shift_kernel<IO, VEC>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_token_shift(const ShiftArgs& a, int dtype, bool vec, hipStream_t s) {
    if (dtype == 0) return vec ? launch_shift_t<float, 4>(a, s) : launch_shift_t<float, 1>(a, s);
    return vec ? launch_shift_t<uint16_t, 8>(a, s) : launch_shift_t<uint16_t, 1>(a, s);
}

}  // namespace wkv
