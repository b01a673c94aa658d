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
// Chunk states along a sequence, two ways (the same floats added in the same order, so the
// same bits):
//  * one pass (one launch, q, k, v read once): chunks (workgroups) take tickets in chunk-major
//    order; a chunk sums its sub-chunk aggregates into the chunk aggregate (phi(K)^T V,
//    sum phi(K)), takes the state entering it from the inclusive state of the chunk before it
//    in its sequence (the plumbing of the WKV chained scan, wkv_chain.h: tagged 64-bit record
//    words, status hints, bounded waits), publishes its own inclusive state, and writes its
//    outputs.  A chunk publishes no aggregate of its own: a state is 1056 words (D = M = 32),
//    so an aggregate record costs as many bytes as the inclusive one, and measured, a chain of
//    inclusive states alone was both faster (150.8 against 155.4 us for 64 float32 sequences of
//    16384, 86.0 against 89.8 us bf16) and moved an eighth fewer bytes than a decoupled
//    look-back over published aggregates.  Inclusive states follow one chain of float32
//    additions in chunk order.
//  * three launches: the chunk aggregates to memory; la_scan_kernel turns them, per sequence
//    and entry, into exclusive prefix sums in chunk order; the outputs from those.  k and v
//    are read twice but no chunk waits for another, which wins for few long sequences.
// In both, the state entering each wave is the chunk's plus the earlier waves' aggregates, in
// wave order, so results are bitwise reproducible.
//
// Order of work in a wave: all of its q, k, v loads are issued first (range-checked buffer
// loads, no branch per row); phi(K) and then V pass through the wave's LDS region into the
// operand layouts; the sub-chunk aggregate and the masked similarities (which need no earlier
// chunk, and stay in registers) are formed before the workgroup waits for the chunk's entering
// state; the outputs follow.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "wkv_chain.h"
#include "wkv_kernels.h"
#include "wkv_rows.h"

namespace wkv {

typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));

constexpr int kLaSub = 32;  // positions per wave

// elu(x) + 1: x + 1 for x > 0, e^x otherwise
__device__ __forceinline__ float elu1(float x) { return x > 0.f ? x + 1.f : ex2(x * kLog2e); }

typedef float f32x4a __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4a __attribute__((ext_vector_type(4)));

// A sub-chunk's rows [0, nv) of W elements as a buffer resource: loads of rows beyond nv
// return zeros (the hardware's range check), so no load needs a branch.
template <typename IO, int W>
__device__ __forceinline__ Rsrc sub_chunk_rows(const IO* src, int nv) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<IO*>(src), (short)0, nv * W * (int)sizeof(IO), 0x00020000);
}

// Rows [0, nv) of a 32 x W block (W elements per row) moved through LDS: each lane loads
// 16-byte runs (four float32 or eight bf16 elements, so a wave reads whole rows) into registers,
// and later stores them into st[32][W + 1] as float, phi applied when `feat`; rows beyond nv are
// zero.  (bf16 runs of 8 against 4 elements: 85.0 against 85.9 us for 64 sequences of 16384,
// the same bits.)
template <typename IO, int W>
struct RowRuns {
    static constexpr int kRunElts = sizeof(IO) == 4 ? 4 : 8;  // 16 bytes per run
    static constexpr int kVpr = W / kRunElts;                // runs per row
    static constexpr int kRuns = kLaSub * kVpr / 64;         // runs per lane
    typedef u32x4a Run;
    Run x[kRuns];

    __device__ __forceinline__ void load(const IO* src, int nv, int lane) {
        const Rsrc rs = sub_chunk_rows<IO, W>(src, nv);
#pragma unroll
        for (int i = 0; i < kRuns; ++i) {
            const int n = lane + 64 * i, t = n / kVpr, c = kRunElts * (n % kVpr);
            const uint32_t off = (uint32_t)((t * W + c) * (int)sizeof(IO));
            x[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kStream);
        }
    }
    __device__ __forceinline__ void store(float* st, int nv, bool feat, int lane) const {
#pragma unroll
        for (int i = 0; i < kRuns; ++i) {
            const int n = lane + 64 * i, t = n / kVpr, c = kRunElts * (n % kVpr);
            float y[kRunElts];
            if constexpr (sizeof(IO) == 4) {
#pragma unroll
                for (int j = 0; j < 4; ++j) y[j] = __uint_as_float(x[i][j]);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    y[2 * j] = bf_lo(x[i][j]);
                    y[2 * j + 1] = bf_hi(x[i][j]);
                }
            }
#pragma unroll
            for (int j = 0; j < kRunElts; ++j) st[t * (W + 1) + c + j] = t < nv ? (feat ? elu1(y[j]) : y[j]) : 0.f;
        }
    }
};

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

// Token map of the two contractions over a sub-chunk's 32 positions (phi(K)^T V and tril(A) V):
// element e of lane group g stands for position 16 (e / 4) + 4 g + e % 4.  These are the
// positions a lane holds as accumulator rows of the two 16-position column blocks of a
// similarity tile computed transposed (phi(K) phi(Q)^T), so the masked similarities feed
// tril(A) V straight from registers.  Any map that both operands share gives the same sum,
// for the float32 and the bfloat16 MFMA shapes alike.
__device__ __forceinline__ int tok_idx(int g, int e) { return 16 * (e / 4) + 4 * g + (e % 4); }

// One region per wave holds in turn the sub-chunk's phi(K) rows, its V rows (staged with 16-byte
// loads, read back in the operand layouts) and its aggregate phi(K)^T V (D x M).
template <int D, int M, int NW>
struct LaShared {  // (the aggregates-only phase uses the same layout)
    static constexpr int kRegion = cmax(kLaSub * cmax(D + 1, M + 1), D * (M + 1));
    float R[NW][kRegion];
    float z[NW][D];         // sub-chunk sums of phi(K)
    float den[NW][kLaSub];  // the denominators: phi(q_t) . z entering the sub-chunk + row sum t
    int ticket;
    int start;              // chunk the look-back folds from
    __device__ __forceinline__ float& S(int w, int d, int m) { return R[w][d * (M + 1) + m]; }
    // record entry e of wave w's aggregate: phi(K)^T V entries, then sum phi(K)
    __device__ __forceinline__ float& entry(int w, int e) { return e < D * M ? S(w, e / M, e % M) : z[w][e - D * M]; }
};

// sum of x over the lanes reached by xor with lo, 2 lo, ..., hi (a butterfly)
__device__ __forceinline__ float sum_lanes(float x, int lo, int hi) {
    for (int m = lo; m <= hi; m <<= 1) x += __shfl_xor(x, m);
    return x;
}

// Records of one sequence: [chunk][slot: 0 aggregate, 1 inclusive][D * M + D words].
struct LaRecs {
    uint64_t* rec;
    uint32_t* status;
    int rec_words;
    uint32_t tag_agg, tag_incl, give_up_word;
    __device__ __forceinline__ uint64_t* word(int chunk, int slot, int e) const {
        return rec + ((size_t)chunk * 2 + slot) * rec_words + e;
    }
};

// The state entering chunk ci (ci >= 1) for this thread's record entries e = threadIdx.x +
// i * threads: wave 0 finds the nearest chunk with a published inclusive state and every chunk
// after it published (find_inclusive); every thread then adds, to that inclusive state, the
// aggregates of the chunks after it, in chunk order.  Chunks publish no aggregates, so the
// search ends at chunk ci - 1 once its inclusive state is out.  False after giving up.
template <int NW, int EPT>
__device__ __forceinline__ bool la_look_back(const LaArgs& a, const LaRecs& R, int ci, int& sh_start, int wid,
                                             int lane, float (&pre)[EPT]) {
    if (wid == 0) {
        const int st = find_inclusive<-1>(R.status, a.n_chunks, ci, lane, R.tag_agg, R.tag_incl, a.ctrl,
                                          R.give_up_word);
        if (lane == 0) sh_start = st;
    }
    __syncthreads();
    const int start = sh_start;
    if (start < 0) return false;
#pragma unroll 1
    for (int c = start; c < ci; ++c) {
        const int slot = c == start ? 1 : 0;
        const uint32_t tag = c == start ? R.tag_incl : R.tag_agg;
        uint64_t wv[EPT];
        for (uint32_t spin = 0;; ++spin) {
            bool good = true;
#pragma unroll
            for (int i = 0; i < EPT; ++i) {
                const int e = threadIdx.x + i * 64 * NW;
                wv[i] = e < R.rec_words ? ld_word(R.word(c, slot, e)) : ((uint64_t)tag << 32);
                good = good && word_tag(wv[i]) == tag;
            }
            if (__all(good)) break;
            if (must_stop(a.ctrl, R.give_up_word, spin)) return raise_give_up(a.ctrl, R.give_up_word, lane);
            __builtin_amdgcn_s_sleep(kPollSleep);
        }
#pragma unroll
        for (int i = 0; i < EPT; ++i) pre[i] = c == start ? word_val(wv[i]) : pre[i] + word_val(wv[i]);
    }
    return true;
}

// An element of q, k or v as float32.
template <typename IO>
__device__ __forceinline__ float la_elt(const IO* p, size_t i) {
    if constexpr (sizeof(IO) == 4)
        return reinterpret_cast<const float*>(p)[i];
    else
        return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(p)[i] << 16);
}

// The state entering chunk ci for this thread's record entries without waiting on any other
// chunk, for a chunk whose look-back gave up or a launch forced onto that path.  The entries
// are independent sums over the chunks before ci, so each thread rebuilds its own: walking
// back from chunk ci - 1, it stops at the first complete inclusive word of its entry (or at
// the sequence start), adding on the way each complete aggregate word, and, for a chunk whose
// word is missing, that chunk's entry summed again from k and v in memory (phi(k_j)[d] v_j[m],
// or phi(k_j)[d] for the sum of phi(K)).  Every word used is validated by its own tag.
template <typename IO, int D, int M, int NW, int EPT>
__device__ __forceinline__ void la_rebuild(const LaArgs& a, const LaRecs& R, int bh, int ci, int chunk_len,
                                           float (&pre)[EPT]) {
    constexpr int REC = D * M + D;
    const bool feat = a.feature != 0;
    const IO* k = static_cast<const IO*>(a.k) + (size_t)bh * a.N * D;
    const IO* v = static_cast<const IO*>(a.v) + (size_t)bh * a.N * M;
#pragma unroll 1
    for (int i = 0; i < EPT; ++i) {
        const int e = threadIdx.x + i * 64 * NW;
        float acc = 0.f;
        if (e < REC) {
            const int d = e < D * M ? e / M : e - D * M, m = e % M;
#pragma unroll 1
            for (int c = ci - 1; c >= 0; --c) {
                const uint64_t wi = ld_word(R.word(c, 1, e));
                if (word_tag(wi) == R.tag_incl) {
                    acc += word_val(wi);
                    break;
                }
                const uint64_t wa = ld_word(R.word(c, 0, e));
                if (word_tag(wa) == R.tag_agg) {
                    acc += word_val(wa);
                    continue;
                }
                const int r0 = c * chunk_len, n = min(chunk_len, a.N - r0);
                float sum = 0.f;
#pragma unroll 1
                for (int j = 0; j < n; ++j) {
                    const float kf = la_elt(k, (size_t)(r0 + j) * D + d);
                    const float ph = feat ? elu1(kf) : kf;
                    sum = e < D * M ? fmaf(ph, la_elt(v, (size_t)(r0 + j) * M + m), sum) : sum + ph;
                }
                acc += sum;
            }
        }
        pre[i] = acc;
    }
}

// PHASE kAggregates: the chunk aggregates into a.agg (first of three launches).  PHASE
// kOutputs: the outputs from the chunk's entering state, read from a.agg after la_scan_kernel
// turned the aggregates into exclusive prefix sums (third launch).  PHASE kOnePass: both, with
// the entering state from the look-back (one launch).
constexpr int kAggregates = 0, kOutputs = 1, kOnePass = 2;

template <typename IO, int D, int M, int NW, int PHASE>
__global__ __launch_bounds__(64 * NW) void la_chunk_kernel(LaArgs a) {
    constexpr int ET = kLaSub / 4, ED = D / 4;  // operand elements per lane: token / feature contractions
    constexpr int CH = kLaSub * NW;
    constexpr int REC = D * M + D;                      // floats of a chunk state
    constexpr int EPT = (REC + 64 * NW - 1) / (64 * NW);  // record entries per thread
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, r = lane & 15;
    __shared__ LaShared<D, M, NW> sh;

    // one pass: chunk-major tickets, so the chunks a chunk waits on hold smaller tickets and
    // are running; otherwise the block index
    int tile = blockIdx.x;
    bool forced = false;
    if constexpr (PHASE == kOnePass) {
        if (threadIdx.x == 0) sh.ticket = (int)atomicAdd(&a.ctrl[kCtrlTicket], 1u);
        __syncthreads();
        tile = (int)remap_ticket((uint32_t)__builtin_amdgcn_readfirstlane(sh.ticket),
                                 (uint32_t)a.BH * (uint32_t)a.n_chunks, a.ctrl, forced);
    }
    const int bh = PHASE == kOnePass ? tile % a.BH : tile / a.n_chunks;
    const int ci = PHASE == kOnePass ? tile / a.BH : tile % a.n_chunks;
    const long t0 = (long)ci * CH + wid * kLaSub;
    const int nv = (int)max(0L, min((long)kLaSub, (long)a.N - t0));
    const long row0 = (long)bh * a.N + min(t0, (long)a.N);
    const IO* q = static_cast<const IO*>(a.q) + row0 * D;
    const IO* k = static_cast<const IO*>(a.k) + row0 * D;
    const IO* v = static_cast<const IO*>(a.v) + row0 * M;
    const bool feat = a.feature != 0;
    auto phi = [&](float x) { return feat ? elu1(x) : x; };

    // ---- every load of the sub-chunk is issued first, in the order of use: K, V, Q.  The phi(K)
    // rows, then the V rows, pass through the wave's region (zero beyond nv) into the operand
    // layouts; Q is read in its operand layout (a lane's elements of a row are runs of 8
    // consecutive features, 16-byte loads) ----
    float* sk = sh.R[wid];  // [32][D + 1], then [32][M + 1]
    RowRuns<IO, D> krows;
    RowRuns<IO, M> vrows;
    krows.load(k, nv, lane);
    vrows.load(v, nv, lane);
    u32x4a xq[2][ED / 8][sizeof(IO) == 4 ? 2 : 1];  // raw q: 8 features per run
    {
        const Rsrc rq = sub_chunk_rows<IO, D>(q, nv);
#pragma unroll
        for (int tI = 0; tI < (PHASE == kAggregates ? 0 : 2); ++tI) {
            const int t = 16 * tI + r;
#pragma unroll
            for (int e8 = 0; e8 < ED; e8 += 8) {
                const uint32_t off = (uint32_t)((t * D + kidx<IO, D>(g, e8)) * (int)sizeof(IO));
#pragma unroll
                for (int h = 0; h < (sizeof(IO) == 4 ? 2 : 1); ++h)
                    xq[tI][e8 / 8][h] = __builtin_amdgcn_raw_buffer_load_b128(rq, off + 16 * h, 0, kStream);
            }
        }
    }
    krows.store(sk, nv, feat, lane);

    // ---- operands: phi(K) as A (rows d, k = t) and V as B (k = t, columns m) ----
    float ka[D / 16][ET], vb[M / 16][ET];
#pragma unroll
    for (int e = 0; e < ET; ++e) {
        const int t = tok_idx(g, e);
#pragma unroll
        for (int dI = 0; dI < D / 16; ++dI) ka[dI][e] = sk[t * (D + 1) + 16 * dI + r];
    }
    // phi(Q) as A (rows t, k = d) and phi(K) as B (k = d, columns t)
    float qa[2][ED], kb[2][ED];
#pragma unroll
    for (int tI = 0; tI < (PHASE == kAggregates ? 0 : 2); ++tI) {
        const int t = 16 * tI + r;
#pragma unroll
        for (int e8 = 0; e8 < ED; e8 += 8) {
            const int d = kidx<IO, D>(g, e8);  // first of 8 consecutive features
            float x8[8];
            if constexpr (sizeof(IO) == 4) {
#pragma unroll
                for (int j = 0; j < 8; ++j) x8[j] = __uint_as_float(xq[tI][e8 / 8][j / 4][j % 4]);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    x8[2 * j] = bf_lo(xq[tI][e8 / 8][0][j]);
                    x8[2 * j + 1] = bf_hi(xq[tI][e8 / 8][0][j]);
                }
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                qa[tI][e8 + j] = t < nv ? phi(x8[j]) : 0.f;
                kb[tI][e8 + j] = sk[t * (D + 1) + d + j];
            }
        }
    }
    // the region's phi(K) rows are all read (LDS accesses of a wave complete in order): V next
    vrows.store(sk, nv, false, lane);
#pragma unroll
    for (int e = 0; e < ET; ++e) {
        const int t = tok_idx(g, e);
#pragma unroll
        for (int mJ = 0; mJ < M / 16; ++mJ) vb[mJ][e] = sk[t * (M + 1) + 16 * mJ + r];
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

    // ---- masked similarities, which need no earlier chunk: tile (cJ, tI) of phi(K) phi(Q)^T
    // leaves in lane (g, r) the entries A(t, c) = phi(q_t) . phi(k_c) for t = 16 tI + r and
    // c = 16 cJ + 4 g + j, which are the lane's operand elements e = 4 cJ + j of row t in
    // tril(A) V; rs[tI] is the row sum of row t ----
    float aa[2][ET], rs[2];
#pragma unroll
    for (int tI = 0; tI < (PHASE == kAggregates ? 0 : 2); ++tI) {
        float s = 0.f;
#pragma unroll
        for (int cJ = 0; cJ < 2; ++cJ) {
            f32x4v acc = {0.f, 0.f, 0.f, 0.f};
            if (cJ <= tI) acc = mma<IO, D>(acc, kb[cJ], qa[tI]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float x = 16 * cJ + 4 * g + j <= 16 * tI + r ? acc[j] : 0.f;
                aa[tI][4 * cJ + j] = x;
                s += x;
            }
        }
        rs[tI] = sum_lanes(s, 16, 32);
    }
    __syncthreads();  // every wave's aggregate is in LDS

    // the chunk aggregate, entry by entry: the sub-chunk aggregates added in wave order
    auto chunk_agg = [&](int e) {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) s += sh.entry(w, e);
        return s;
    };
    float* agg = a.agg + ((size_t)bh * a.n_chunks + ci) * REC;
    if constexpr (PHASE == kAggregates) {
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            const int e = threadIdx.x + i * 64 * NW;
            if (e < REC) agg[e] = chunk_agg(e);
        }
        return;
    }

    // ---- the state entering the chunk: the exclusive prefix in a.agg (three launches), or by
    // the chain (one pass: publish the chunk aggregate, look back, publish the inclusive state) ----
    float pre[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int e = threadIdx.x + i * 64 * NW;
        pre[i] = PHASE == kOutputs && e < REC ? agg[e] : 0.f;
    }
    uint32_t epoch = 0;
    if constexpr (PHASE == kOnePass) {
        epoch = __builtin_amdgcn_readfirstlane(a.ctrl[kCtrlEpoch]);  // constant during the launch
        LaRecs recs;
        recs.rec = static_cast<uint64_t*>(a.recs) + (size_t)bh * a.n_chunks * 2 * REC;
        recs.status = a.status + (size_t)bh * a.n_chunks;
        recs.rec_words = REC;
        recs.tag_agg = (epoch << 2) | kKindAgg;
        recs.tag_incl = (epoch << 2) | kKindIncl;
        recs.give_up_word = epoch | kCtrlGiveUpMark;
        const bool has_next = ci + 1 < a.n_chunks;
        forced = forced || launch_forced(a.ctrl);
        if (ci > 0) {
            bool have = false;
            if (!forced) {
                have = la_look_back<NW, EPT>(a, recs, ci, sh.start, wid, lane, pre);
            } else {
                raise_give_up(a.ctrl, recs.give_up_word, lane);
            }
            if (!have) la_rebuild<IO, D, M, NW, EPT>(a, recs, bh, ci, CH, pre);
        }
        if (has_next) {
#pragma unroll
            for (int i = 0; i < EPT; ++i) {
                const int e = threadIdx.x + i * 64 * NW;
                if (e < REC) st_word(recs.word(ci, 1, e), pre[i] + chunk_agg(e), recs.tag_incl);
            }
            if (threadIdx.x == 0)
                __hip_atomic_store(&recs.status[ci], recs.tag_incl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    // the state entering each wave: the chunk's plus the waves before, in wave order, replacing
    // the sub-chunk aggregates in place
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int e = threadIdx.x + i * 64 * NW;
        if (e < REC) {
            float run = pre[i];
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                float& x = sh.entry(w, e);
                const float dx = x;
                x = run;
                run += dx;
            }
        }
    }
    __syncthreads();
    float zb[ED];  // z entering the wave as B operand (k = d)
#pragma unroll
    for (int e = 0; e < ED; ++e) zb[e] = sh.z[wid][kidx<IO, D>(g, e)];
    // the denominators phi(q_t) . z + row sum for the rows t = 16 tI + r; the outputs read them
    // back in accumulator rows (written and read by this wave only)
#pragma unroll
    for (int tI = 0; tI < 2; ++tI) {
        float p = 0.f;
#pragma unroll
        for (int e = 0; e < ED; ++e) p = fmaf(qa[tI][e], zb[e], p);
        p = sum_lanes(p, 16, 32);
        if (g == 0) sh.den[wid][16 * tI + r] = p + rs[tI];
    }

    // ---- outputs: (tril(A) V + phi(Q) S_w) / den ----
    IO* out = static_cast<IO*>(a.out) + row0 * M;
    float inv[2][4];
#pragma unroll
    for (int tI = 0; tI < 2; ++tI)
#pragma unroll
        for (int j = 0; j < 4; ++j) inv[tI][j] = 1.f / sh.den[wid][16 * tI + 4 * g + j];
#pragma unroll
    for (int mJ = 0; mJ < M / 16; ++mJ) {
        float sb[ED];  // S_w columns 16 mJ ... as B operand (k = d)
#pragma unroll
        for (int e = 0; e < ED; ++e) sb[e] = sh.S(wid, kidx<IO, D>(g, e), 16 * mJ + r);
#pragma unroll
        for (int tI = 0; tI < 2; ++tI) {
            f32x4v acc = {0.f, 0.f, 0.f, 0.f};
            acc = mma<IO, kLaSub>(acc, aa[tI], vb[mJ]);
            acc = mma<IO, D>(acc, qa[tI], sb);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * tI + 4 * g + j, col = 16 * mJ + r;
                if (row < nv) {
                    const float y = acc[j] * inv[tI][j];
                    if constexpr (sizeof(IO) == 4)
                        reinterpret_cast<float*>(out)[row * M + col] = y;
                    else
                        reinterpret_cast<uint16_t*>(out)[row * M + col] = (uint16_t)(pack_bf16(y, 0.f) & 0xffffu);
                }
            }
        }
    }

    // ---- launch bookkeeping: the last workgroup to finish prepares the next launch ----
    if constexpr (PHASE == kOnePass) {
        __syncthreads();
        if (threadIdx.x == 0) finish_tile(a.ctrl, (uint32_t)a.BH * (uint32_t)a.n_chunks, epoch, false);
    }
    (void)CH;
}

// Per (sequence, record entry): the chunk aggregates replaced by their exclusive prefix sums,
// in chunk order (the second of three launches).
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
    if (a.one_pass) {
        hipLaunchKernelGGL((la_chunk_kernel<IO, D, M, NW, kOnePass>), dim3(blocks), dim3(64 * NW), 0, s, a);
    } else {
        hipLaunchKernelGGL((la_chunk_kernel<IO, D, M, NW, kAggregates>), dim3(blocks), dim3(64 * NW), 0, s, a);
        hipLaunchKernelGGL(la_scan_kernel, dim3((unsigned)(((long)a.BH * (D * M + D) + 255) / 256)), dim3(256), 0,
                           s, a, D * M + D);
        hipLaunchKernelGGL((la_chunk_kernel<IO, D, M, NW, kOutputs>), dim3(blocks), dim3(64 * NW), 0, s, a);
    }
    return hipGetLastError();
}

// Positions per chunk: 16 waves of 32 for D = M = 32 (one 1024-thread workgroup per CU: the
// chain of inclusive states is half as long and its records weigh half as much per byte of
// q, k, v, out as with 8 waves); 8 waves when D or M is 64 (one workgroup per CU either way for
// D = M = 64, its LDS and registers being twice as large).
int la_chunk_len(int D, int M, int dtype) { (void)dtype; return kLaSub * (D * M <= 1024 ? 16 : 8); }

hipError_t launch_linear_attention(const LaArgs& a, int dtype, hipStream_t s) {
    if (a.D == 32 && a.M == 32)
        return dtype == 0 ? launch_la_t<float, 32, 32, 16>(a, s) : launch_la_t<uint16_t, 32, 32, 16>(a, s);
    if (a.D == 64 && a.M == 64)
        return dtype == 0 ? launch_la_t<float, 64, 64, 8>(a, s) : launch_la_t<uint16_t, 64, 64, 8>(a, s);
    if (a.D == 32 && a.M == 64)
        return dtype == 0 ? launch_la_t<float, 32, 64, 8>(a, s) : launch_la_t<uint16_t, 32, 64, 8>(a, s);
    if (a.D == 64 && a.M == 32)
        return dtype == 0 ? launch_la_t<float, 64, 32, 8>(a, s) : launch_la_t<uint16_t, 64, 32, 8>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace wkv
