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
