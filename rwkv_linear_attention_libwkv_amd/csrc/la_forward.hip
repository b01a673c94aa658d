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
// aggregates, adds them in wave order to the chunk's entering state, and writes the outputs.
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

// acc += A (16 x K) B (K x 16) for this lane's tile slot: fa(i, k) and fb(k, n) give the
// operands; lane (g = lane / 16, r = lane % 16) supplies row i = r of A and column n = r of B.
// float32: 16x16x4 steps; group g takes the k block [g K/4, (g+1) K/4) one k per step.
// bfloat16: 16x16x32 steps; group g takes k = 32 s + 8 g + j, j < 8.
template <typename IO, int K, typename FA, typename FB>
__device__ __forceinline__ f32x4v tile_mma(f32x4v acc, int lane, FA fa, FB fb) {
    const int g = lane >> 4, r = lane & 15;
    if constexpr (sizeof(IO) == 4) {
        static_assert(K % 4 == 0, "K");
#pragma unroll
        for (int s = 0; s < K / 4; ++s) {
            const int k = g * (K / 4) + s;
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa(r, k), fb(k, r), acc, 0, 0, 0);
        }
    } else {
        static_assert(K % 32 == 0, "K");
#pragma unroll
        for (int s = 0; s < K / 32; ++s) {
            bf16x8v a, b;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int k = 32 * s + 8 * g + j;
                a[j] = (__bf16)fa(r, k);
                b[j] = (__bf16)fb(k, r);
            }
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
        }
    }
    return acc;
}

template <int D, int M, int NW>
struct LaShared {
    float S[NW][D][M + 1];  // sub-chunk aggregates, then each wave's entering state
    float z[NW][D];
    float A[NW][kLaSub][kLaSub + 1];  // masked similarities of each sub-chunk
    float den[NW][kLaSub];
};

// PHASE 0: chunk aggregates into a.agg.  PHASE 1: outputs from the chunk's entering state.
template <typename IO, int D, int M, int NW, int PHASE>
__global__ __launch_bounds__(64 * NW) void la_chunk_kernel(LaArgs a) {
    constexpr int CH = kLaSub * NW;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, r = lane & 15;
    __shared__ LaShared<D, M, NW> sh;

    const int bh = blockIdx.x / a.n_chunks;
    const int ci = blockIdx.x % a.n_chunks;
    const long t0 = (long)ci * CH + wid * kLaSub;
    const int nv = (int)max(0L, min((long)kLaSub, (long)a.N - t0));
    const long row0 = (long)bh * a.N + min(t0, (long)a.N);
    const IO* q = static_cast<const IO*>(a.q) + row0 * D;
    const IO* k = static_cast<const IO*>(a.k) + row0 * D;
    const IO* v = static_cast<const IO*>(a.v) + row0 * M;
    const bool feat = a.feature != 0;

    // rows at or beyond nv contribute nothing (phi(k) = 0 and v = 0 there)
    auto phik = [&](int t, int d) -> float {
        if (t >= nv) return 0.f;
        const float x = ld<IO>(k + t * D + d);
        return feat ? elu1(x) : x;
    };
    auto phiq = [&](int t, int d) -> float {
        if (t >= nv) return 0.f;
        const float x = ld<IO>(q + t * D + d);
        return feat ? elu1(x) : x;
    };
    auto val = [&](int t, int m) -> float { return t < nv ? ld<IO>(v + t * M + m) : 0.f; };

    // ---- this sub-chunk's aggregate phi(K)^T V (D x M) and sum phi(K) ----
#pragma unroll
    for (int dI = 0; dI < D / 16; ++dI)
#pragma unroll
        for (int mJ = 0; mJ < M / 16; ++mJ) {
            f32x4v acc = {0.f, 0.f, 0.f, 0.f};
            acc = tile_mma<IO, kLaSub>(acc, lane, [&](int i, int t) { return phik(t, 16 * dI + i); },
                                       [&](int t, int n) { return val(t, 16 * mJ + n); });
#pragma unroll
            for (int j = 0; j < 4; ++j) sh.S[wid][16 * dI + 4 * g + j][16 * mJ + r] = acc[j];
        }
    for (int d = lane; d < D; d += 64) {
        float s = 0.f;
        for (int t = 0; t < nv; ++t) s += phik(t, d);
        sh.z[wid][d] = s;
    }
    __syncthreads();

    const size_t rec = (size_t)D * M + D;  // floats per chunk record
    float* agg = a.agg + ((size_t)bh * a.n_chunks + ci) * rec;
    if constexpr (PHASE == 0) {
        // chunk aggregate: the sub-chunk aggregates added in wave order
        for (int e = threadIdx.x; e < (int)rec; e += 64 * NW) {
            float s = 0.f;
            for (int w = 0; w < NW; ++w) s += e < D * M ? sh.S[w][e / M][e % M] : sh.z[w][e - D * M];
            agg[e] = s;
        }
        return;
    } else {
        // ---- each wave's entering state: the chunk's (exclusive prefix) plus the waves before ----
        constexpr int PER = (D * M + 63) / 64;
        float st[PER];
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int e = lane + 64 * p;
            float s = 0.f;
            if (e < D * M) {
                s = agg[e];
                for (int w = 0; w < wid; ++w) s += sh.S[w][e / M][e % M];
            }
            st[p] = s;
        }
        float zs = 0.f;
        if (lane < D) {
            zs = agg[D * M + lane];
            for (int w = 0; w < wid; ++w) zs += sh.z[w][lane];
        }
        __syncthreads();  // every wave has read the aggregates
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int e = lane + 64 * p;
            if (e < D * M) sh.S[wid][e / M][e % M] = st[p];
        }
        if (lane < D) sh.z[wid][lane] = zs;

        // ---- masked similarities phi(Q) phi(K)^T (32 x 32) ----
#pragma unroll
        for (int tI = 0; tI < 2; ++tI)
#pragma unroll
            for (int tJ = 0; tJ < 2; ++tJ) {
                f32x4v acc = {0.f, 0.f, 0.f, 0.f};
                if (tJ <= tI)
                    acc = tile_mma<IO, D>(acc, lane, [&](int i, int d) { return phiq(16 * tI + i, d); },
                                          [&](int d, int n) { return phik(16 * tJ + n, d); });
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int row = 16 * tI + 4 * g + j, col = 16 * tJ + r;
                    sh.A[wid][row][col] = col <= row ? acc[j] : 0.f;
                }
            }
        __syncthreads();
        // denominators, one position per lane
        if (lane < kLaSub) {
            float s = 0.f;
            for (int c = 0; c <= lane; ++c) s += sh.A[wid][lane][c];
            for (int d = 0; d < D; ++d) s = fmaf(phiq(lane, d), sh.z[wid][d], s);
            sh.den[wid][lane] = s;
        }
        __syncthreads();

        // ---- outputs: (tril(A) V + phi(Q) S_w) / den ----
        IO* out = static_cast<IO*>(a.out) + row0 * M;
#pragma unroll
        for (int tI = 0; tI < 2; ++tI)
#pragma unroll
            for (int mJ = 0; mJ < M / 16; ++mJ) {
                f32x4v acc = {0.f, 0.f, 0.f, 0.f};
                acc = tile_mma<IO, kLaSub>(acc, lane, [&](int i, int t) { return sh.A[wid][16 * tI + i][t]; },
                                           [&](int t, int n) { return val(t, 16 * mJ + n); });
                acc = tile_mma<IO, D>(acc, lane, [&](int i, int d) { return phiq(16 * tI + i, d); },
                                      [&](int d, int n) { return sh.S[wid][d][16 * mJ + n]; });
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int row = 16 * tI + 4 * g + j, col = 16 * mJ + r;
                    if (row < nv) {
                        const float y = acc[j] / sh.den[wid][row];
                        if constexpr (sizeof(IO) == 4)
                            reinterpret_cast<float*>(out)[row * M + col] = y;
                        else
                            reinterpret_cast<uint16_t*>(out)[row * M + col] = (uint16_t)(pack_bf16(y, 0.f) & 0xffffu);
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
    for (int c = 0; c < a.n_chunks; ++c) {
        const float x = p[(size_t)c * rec];
        p[(size_t)c * rec] = run;
        run += x;
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
