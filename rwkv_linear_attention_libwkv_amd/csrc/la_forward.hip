// Causal linear attention for gfx950, on the matrix cores.
//
// Page "Transformers are RNNs: 선형 어텐션으로 만드는 빠른 자기회귀 트랜스포머", sections
// "인과 마스킹과 누적합" and "특징 맵 선택과 계산 비용": for one sequence (batch-head),
//   out_i = phi(q_i)^T S_i / (phi(q_i)^T z_i),  S_i = sum_{j<=i} phi(k_j) v_j^T,  z_i = sum_{j<=i} phi(k_j),
// with phi(x) = elu(x) + 1 (or q, k used as given).
//
// Chunked evaluation.  A chunk of CH = 32 NW positions is split into NW sub-chunks of 32, one
// per wave.  With S_w, z_w the state entering sub-chunk w,
//   out_t = (phi(Q) S_w + tril(phi(Q) phi(K)^T) V)_t / (phi(Q) z_w + rowsum tril(phi(Q) phi(K)^T))_t,
// and S_{w+1} = S_w + phi(K)^T V, z_{w+1} = z_w + sum_t phi(K_t) (sums over the sub-chunk).
// Every product is a dense 16 x 16 tile contraction on MFMA: v_mfma_f32_16x16x4_f32 for float32
// inputs, v_mfma_f32_16x16x32_bf16 for bfloat16 inputs (phi, the masked similarities and the
// entering state rounded to bf16 as operands; float32 accumulation).
//
// Three launches: la_chunk_kernel<0> writes each chunk's aggregate (phi(K)^T V, sum phi(K));
// la_scan_kernel turns them, per sequence and entry, into the exclusive prefix (the state
// entering each chunk, summed in chunk order); la_chunk_kernel<1> recomputes the sub-chunk
// aggregates, adds them in wave order to the chunk's entering state (each workgroup thread
// taking a slice of the entries), and writes the outputs.
// Every sum has a fixed order, so results are bitwise reproducible.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wkv_kernels.h"
#include "wkv_rows.h"

namespace wkv {

typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));

constexpr int kLaSub = 32;  // positions per wave

// elu(x) + 1: x + 1 for x > 0, e^x otherwise
__device__ __forceinline__ float elu1(float x) { return x > 0.f ? x + 1.f : ex2(x * kLog2e); }

template <typename IO>
__device__ __forceinline__ float ld(const IO* p) {
    if constexpr (sizeof(IO) == 4)
        return *reinterpret_cast<const float*>(p);
    else
        return bf_lo((uint32_t)*reinterpret_cast<const uint16_t*>(p));
}

// Eight consecutive elements (32 or 16 bytes, aligned) as floats; zeros when !ok.
typedef float f32x4a __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4a __attribute__((ext_vector_type(4)));
template <typename IO>
__device__ __forceinline__ void load8(const IO* p, bool ok, float (&x)[8]) {
    if constexpr (sizeof(IO) == 4) {
        f32x4a a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
        if (ok) {
            a = *reinterpret_cast<const f32x4a*>(p);
            b = *reinterpret_cast<const f32x4a*>(p + 4);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[j] = a[j];
            x[4 + j] = b[j];
        }
    } else {
        u32x4a a = {0u, 0u, 0u, 0u};
        if (ok) a = *reinterpret_cast<const u32x4a*>(p);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[2 * j] = bf_lo(a[j]);
            x[2 * j + 1] = bf_hi(a[j]);
        }
    }
}

// Rows [0, nv) of a 32 x W block (W elements per row, from src) into st[32][W + 1] as float,
// phi applied when `feat`; rows beyond nv are zero.  Each lane moves runs of four elements
// (16-byte float32 or 8-byte bf16 loads), so a wave reads whole rows.
template <typename IO, int W>
__device__ __forceinline__ void stage_rows(const IO* src, int nv, float* st, bool feat, int lane) {
    constexpr int VPR = W / 4;  // runs per row
#pragma unroll
    for (int i = lane; i < kLaSub * VPR; i += 64) {
        const int t = i / VPR, c = 4 * (i % VPR);
        float x[4] = {0.f, 0.f, 0.f, 0.f};
        if (t < nv) {
            if constexpr (sizeof(IO) == 4) {
                const f32x4a a = *reinterpret_cast<const f32x4a*>(src + t * W + c);
#pragma unroll
                for (int j = 0; j < 4; ++j) x[j] = feat ? elu1(a[j]) : a[j];
            } else {
                typedef uint32_t u32x2a __attribute__((ext_vector_type(2)));
                const u32x2a a = *reinterpret_cast<const u32x2a*>(src + t * W + c);
                x[0] = bf_lo(a[0]);
                x[1] = bf_hi(a[0]);
                x[2] = bf_lo(a[1]);
                x[3] = bf_hi(a[1]);
                if (feat)
#pragma unroll
                    for (int j = 0; j < 4; ++j) x[j] = elu1(x[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) st[t * (W + 1) + c + j] = x[j];
    }
}

// Operands of a 16 x 16 x K tile product held in registers: each lane keeps K/4 elements of
// its A row (i = lane % 16) and of its B column (n = lane % 16).  Element e of lane group
// g = lane / 16 stands for k = kidx(g, e): float32 (16x16x4 steps, one k per step) uses the
// block [g K/4, (g+1) K/4); bfloat16 (16x16x32 steps, eight k per step) uses
// k = 32 (e / 8) + 8 g + e % 8.  Both A and B use the same map, so the products pair up;
// the map makes a lane's q and k elements contiguous in memory.
template <typename IO, int K>
__device__ __forceinline__ int kidx(int g, int e) {
    if constexpr (sizeof(IO) == 4)
        return g * (K / 4) + e;
    else
        return 32 * (e / 8) + 8 * g + (e % 8);
}

template <typename IO, int K>
__device__ __forceinline__ f32x4v mma(f32x4v acc, const float (&x)[K / 4], const float (&y)[K / 4]) {
    if constexpr (sizeof(IO) == 4) {
#pragma unroll
        for (int e = 0; e < K / 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x[e], y[e], acc, 0, 0, 0);
    } else {
#pragma unroll
        for (int s = 0; s < K / 32; ++s) {
            bf16x8v a, b;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                a[j] = (__bf16)x[8 * s + j];
                b[j] = (__bf16)y[8 * s + j];
            }
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
        }
    }
    return acc;
}

constexpr int cmax(int a, int b) { return a > b ? a : b; }

// One region per wave holds in turn the sub-chunk's phi(K) and V rows (staged with 16-byte
// loads, read back in the operand layouts), its aggregate phi(K)^T V (D x M) and, once every
// wave has read the aggregates it needs, the masked similarities (32 x 32).
template <int D, int M, int NW, int PHASE>
struct LaShared {
    static constexpr int kRegion =
        cmax(kLaSub * (D + 1) + kLaSub * (M + 1), cmax(D * (M + 1), kLaSub * (kLaSub + 1)));
    float R[NW][kRegion];
    float z[NW][D];                       // sub-chunk sums of phi(K)
    float den[PHASE ? NW : 1][kLaSub];    // phi(q_t) . z entering the sub-chunk
    __device__ __forceinline__ float& S(int w, int d, int m) { return R[w][d * (M + 1) + m]; }
    __device__ __forceinline__ float& A(int w, int t, int c) { return R[w][t * (kLaSub + 1) + c]; }
};

// sum of x over the lanes reached by xor with lo, 2 lo, ..., hi (a butterfly)
__device__ __forceinline__ float sum_lanes(float x, int lo, int hi) {
    for (int m = lo; m <= hi; m <<= 1) x += __shfl_xor(x, m);
    return x;
}

// PHASE 0: chunk aggregates into a.agg.  PHASE 1: outputs from the chunk's entering state.
template <typename IO, int D, int M, int NW, int PHASE>
__global__ __launch_bounds__(64 * NW) void la_chunk_kernel(LaArgs a) {
    constexpr int CH = kLaSub * NW;
    constexpr int ET = kLaSub / 4, ED = D / 4;  // operand elements per lane: token / feature contractions
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, r = lane & 15;
    __shared__ LaShared<D, M, NW, PHASE> sh;

    const int bh = blockIdx.x / a.n_chunks;
    const int ci = blockIdx.x % a.n_chunks;
    const long t0 = (long)ci * CH + wid * kLaSub;
    const int nv = (int)max(0L, min((long)kLaSub, (long)a.N - t0));
    const long row0 = (long)bh * a.N + min(t0, (long)a.N);
    const IO* q = static_cast<const IO*>(a.q) + row0 * D;
    const IO* k = static_cast<const IO*>(a.k) + row0 * D;
    const IO* v = static_cast<const IO*>(a.v) + row0 * M;
    const bool feat = a.feature != 0;
    auto phi = [&](float x) { return feat ? elu1(x) : x; };

    // ---- stage this sub-chunk's phi(K) and V rows in the wave's region (zero beyond nv) ----
    float* sk = sh.R[wid];                      // [32][D + 1]
    float* sv = sh.R[wid] + kLaSub * (D + 1);   // [32][M + 1]
    stage_rows<IO, D>(k, nv, sk, feat, lane);
    stage_rows<IO, M>(v, nv, sv, false, lane);

    // ---- operands: phi(K) as A (rows d, k = t) and V as B (k = t, columns m) ----
    float ka[D / 16][ET], vb[M / 16][ET];
#pragma unroll
    for (int e = 0; e < ET; ++e) {
        const int t = kidx<IO, kLaSub>(g, e);
#pragma unroll
        for (int dI = 0; dI < D / 16; ++dI) ka[dI][e] = sk[t * (D + 1) + 16 * dI + r];
#pragma unroll
        for (int mJ = 0; mJ < M / 16; ++mJ) vb[mJ][e] = sv[t * (M + 1) + 16 * mJ + r];
    }
    // phi(Q) as A (rows t, k = d; from memory: a lane's elements of a row are runs of 8
    // consecutive features, read with 16-byte loads) and phi(K) as B (k = d, columns t)
    float qa[2][ED], kb[2][ED];
    if constexpr (PHASE == 1) {
#pragma unroll
        for (int tI = 0; tI < 2; ++tI) {
            const int t = 16 * tI + r;
#pragma unroll
            for (int e8 = 0; e8 < ED; e8 += 8) {
                const int d = kidx<IO, D>(g, e8);  // first of 8 consecutive features
                float xq[8];
                load8<IO>(q + t * D + d, t < nv, xq);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    qa[tI][e8 + j] = t < nv ? phi(xq[j]) : 0.f;
                    kb[tI][e8 + j] = sk[t * (D + 1) + d + j];
                }
            }
        }
    }

    // ---- sub-chunk aggregate phi(K)^T V and sum phi(K) ----
#pragma unroll
    for (int dI = 0; dI < D / 16; ++dI) {
#pragma unroll
        for (int mJ = 0; mJ < M / 16; ++mJ) {
            f32x4v acc = {0.f, 0.f, 0.f, 0.f};
            acc = mma<IO, kLaSub>(acc, ka[dI], vb[mJ]);
#pragma unroll
            for (int j = 0; j < 4; ++j) sh.S(wid, 16 * dI + 4 * g + j, 16 * mJ + r) = acc[j];
        }
        float zs = 0.f;
#pragma unroll
        for (int e = 0; e < ET; ++e) zs += ka[dI][e];
        zs = sum_lanes(zs, 16, 32);
        if (g == 0) sh.z[wid][16 * dI + r] = zs;
    }

    const size_t rec = (size_t)D * M + D;  // floats per chunk record
    float* agg = a.agg + ((size_t)bh * a.n_chunks + ci) * rec;
    if constexpr (PHASE == 0) {
        __syncthreads();
        // chunk aggregate: the sub-chunk aggregates added in wave order
        for (int e = threadIdx.x; e < (int)rec; e += 64 * NW) {
            float s = 0.f;
            for (int w = 0; w < NW; ++w) s += e < D * M ? sh.S(w, e / M, e % M) : sh.z[w][e - D * M];
            agg[e] = s;
        }
    } else {
        __syncthreads();  // every wave's aggregate is in LDS

        // ---- the state entering each wave: the chunk's plus the waves before, in wave order;
        // the entries are split across all the workgroup's threads and replaced in place ----
        for (int e = threadIdx.x; e < (int)rec; e += 64 * NW) {
            float run = agg[e];
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                float& x = e < D * M ? sh.S(w, e / M, e % M) : sh.z[w][e - D * M];
                const float dx = x;
                x = run;
                run += dx;
            }
        }
        __syncthreads();
        float sb[M / 16][ED], zb[ED];  // as B operand (k = d, columns m)
#pragma unroll
        for (int e = 0; e < ED; ++e) {
            const int d = kidx<IO, D>(g, e);
#pragma unroll
            for (int mJ = 0; mJ < M / 16; ++mJ) sb[mJ][e] = sh.S(wid, d, 16 * mJ + r);
            zb[e] = sh.z[wid][d];
        }
        // phi(q_t) . z for the rows t = 16 tI + r
#pragma unroll
        for (int tI = 0; tI < 2; ++tI) {
            float p = 0.f;
#pragma unroll
            for (int e = 0; e < ED; ++e) p = fmaf(qa[tI][e], zb[e], p);
            p = sum_lanes(p, 16, 32);
            if (g == 0) sh.den[wid][16 * tI + r] = p;
        }
        __syncthreads();  // every wave has read the aggregates: the regions take the similarities

        // ---- masked similarities phi(Q) phi(K)^T (32 x 32) and their row sums ----
        float rs[2][4];
#pragma unroll
        for (int tI = 0; tI < 2; ++tI) {
#pragma unroll
            for (int j = 0; j < 4; ++j) rs[tI][j] = 0.f;
#pragma unroll
            for (int tJ = 0; tJ < 2; ++tJ) {
                f32x4v acc = {0.f, 0.f, 0.f, 0.f};
                if (tJ <= tI) acc = mma<IO, D>(acc, qa[tI], kb[tJ]);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int row = 16 * tI + 4 * g + j, col = 16 * tJ + r;
                    const float x = col <= row ? acc[j] : 0.f;
                    sh.A(wid, row, col) = x;
                    rs[tI][j] += x;
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) rs[tI][j] = sum_lanes(rs[tI][j], 1, 8);
        }
        __syncthreads();

        // ---- outputs: (tril(A) V + phi(Q) S_w) / den ----
        IO* out = static_cast<IO*>(a.out) + row0 * M;
#pragma unroll
        for (int tI = 0; tI < 2; ++tI) {
            float aa[ET], inv[4];
#pragma unroll
            for (int e = 0; e < ET; ++e) aa[e] = sh.A(wid, 16 * tI + r, kidx<IO, kLaSub>(g, e));
#pragma unroll
            for (int j = 0; j < 4; ++j) inv[j] = 1.f / (rs[tI][j] + sh.den[wid][16 * tI + 4 * g + j]);
#pragma unroll
            for (int mJ = 0; mJ < M / 16; ++mJ) {
                f32x4v acc = {0.f, 0.f, 0.f, 0.f};
                acc = mma<IO, kLaSub>(acc, aa, vb[mJ]);
                acc = mma<IO, D>(acc, qa[tI], sb[mJ]);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int row = 16 * tI + 4 * g + j, col = 16 * mJ + r;
                    if (row < nv) {
                        const float y = acc[j] * inv[j];
                        if constexpr (sizeof(IO) == 4)
                            reinterpret_cast<float*>(out)[row * M + col] = y;
                        else
                            reinterpret_cast<uint16_t*>(out)[row * M + col] = (uint16_t)(pack_bf16(y, 0.f) & 0xffffu);
                    }
                }
            }
        }
    }
}

// Per (sequence, record entry): the chunk aggregates replaced by their exclusive prefix sums,
// in chunk order.
__global__ __launch_bounds__(256) void la_scan_kernel(LaArgs a, int rec) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= (long)a.BH * rec) return;
    const long bh = i / rec, e = i % rec;
    float* p = a.agg + (size_t)bh * a.n_chunks * rec + e;
    float run = 0.f;
    // eight chunks' loads in flight at a time; the sums stay in chunk order
    for (int c0 = 0; c0 < a.n_chunks; c0 += 8) {
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = c0 + j < a.n_chunks ? p[(size_t)(c0 + j) * rec] : 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (c0 + j < a.n_chunks) p[(size_t)(c0 + j) * rec] = run;
            run += x[j];
        }
    }
}

template <typename IO, int D, int M, int NW>
static hipError_t launch_la_t(const LaArgs& a, hipStream_t s) {
    const unsigned blocks = (unsigned)((long)a.BH * a.n_chunks);
    const int rec = D * M + D;
    hipLaunchKernelGGL((la_chunk_kernel<IO, D, M, NW, 0>), dim3(blocks), dim3(64 * NW), 0, s, a);
    hipLaunchKernelGGL(la_scan_kernel, dim3((unsigned)(((long)a.BH * rec + 255) / 256)), dim3(256), 0, s, a, rec);
    hipLaunchKernelGGL((la_chunk_kernel<IO, D, M, NW, 1>), dim3(blocks), dim3(64 * NW), 0, s, a);
    return hipGetLastError();
}

int la_chunk_len(int D, int M) { return kLaSub * (D * M <= 1024 ? 8 : 4); }

hipError_t launch_linear_attention(const LaArgs& a, int dtype, hipStream_t s) {
    if (a.D == 32 && a.M == 32)
        return dtype == 0 ? launch_la_t<float, 32, 32, 8>(a, s) : launch_la_t<uint16_t, 32, 32, 8>(a, s);
    if (a.D == 64 && a.M == 64)
        return dtype == 0 ? launch_la_t<float, 64, 64, 4>(a, s) : launch_la_t<uint16_t, 64, 64, 4>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace wkv
