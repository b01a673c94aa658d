// Whole-sequence WKV forward kernels for gfx950.
//
// Operator: page "Reinventing RNNs for the Transformer Era: RWKV" (velog review),
// section "WKV 연산자" (WKV equation) and section "RNN-유사추론" (RNN form).  The
// page's time-parallel training mode (section "Transformer-유사학습") runs every
// other op over batch and time at once and only WKV "as a scan"; the two kernels
// here are that scan.
//
// Layout: k, v, y are [B, T, C] with C fastest.  Every thread owns one channel of one
// batch row and a wave owns 64 consecutive channels, so a wave reads one contiguous
// segment of a time step per load.
//
//  * fwd_seq_kernel: each thread walks all T for its channel, L tokens at a time
//    (the chunk fast path of wkv_device.h with a per-chunk reference).
//  * fwd_chunked_kernel: single pass over HBM.  A workgroup of NW waves owns one
//    tile = 64 channels x (NW*L tokens); every wave keeps its L tokens of k, v in
//    registers, reduces them to a per-wave state, the waves are combined in LDS into
//    the tile's aggregate, and the tile's incoming state is read from the previous
//    tile's inclusive record when that has already been published, else obtained from
//    the tiles before it by a decoupled look-back over published per-tile states (the
//    chained-scan technique of Merrill and Garland, "Single-pass Parallel Prefix Scan
//    with Decoupled Look-back", 2016).  Each wave then produces its outputs from its
//    registers, so k and v are read once and y written once.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "wkv_device.h"
#include "wkv_kernels.h"
#include "wkv_chain.h"
#include "wkv_rows.h"

namespace wkv {

// ----------------------------------------------------------------------------
// A wave's chunk: L consecutive tokens of k and v of this lane's channel, in registers.
//
// Fast path for a full, well-conditioned chunk with reference R (log2 units):
//   x_j = 2^(k_j log2e - R),  y_j = (A/2^R + e^u x_j v_j)/(B/2^R + e^u x_j),  A/2^R <- d A/2^R + x_j v_j
// (and B likewise), with y_j formed as fma(e^u, x_j v_j, A/2^R) * rcp(fma(e^u, x_j, B/2^R)).
// aggregate() gives the state of the chunk's tokens from the empty state; outputs()
// gives the outputs from the state entering the chunk and returns the state after it.
// ----------------------------------------------------------------------------

// Load L rows of k and v in row-pair mode into packed words (word j: tokens 2j, 2j+1 of
// this lane's channel).  Rows at or beyond nv and lanes with !valid read as zero.
template <int L>
__device__ __forceinline__ void load_pairs(const WaveRows& w, int nv, bool valid, uint32_t (&k)[L / 2],
                                           uint32_t (&v)[L / 2]) {
    // every load is issued before the first exchange (which waits for its operand),
    // and all 64 lanes reach the exchanges: only the loads are predicated
    uint32_t xk[L / 2], xv[L / 2];
#pragma unroll
    for (int jj = 0; jj < L / 2; ++jj) {
        xk[jj] = 0u;
        xv[jj] = 0u;
        if (valid && 2 * jj + (int)w.upper < nv) {
            const uint32_t so = (uint32_t)(2 * jj) * w.row_bytes;
            xk[jj] = __builtin_amdgcn_raw_buffer_load_b32(w.k, w.pair_off, so, kStream);
            xv[jj] = __builtin_amdgcn_raw_buffer_load_b32(w.v, w.pair_off, so, kStream);
        }
    }
    const uint32_t sel = pair_sel(w.upper);
#pragma unroll
    for (int jj = 0; jj < L / 2; ++jj) {
        k[jj] = pair_exchange(xk[jj], w.partner, sel);
        v[jj] = pair_exchange(xv[jj], w.partner, sel);
        // at most eight exchanges in flight, each completed in place: issuing all of
        // them first (or sinking the byte picks to their first use) would hold a
        // second register for every loaded word
        if (jj % 4 == 3) {
#pragma unroll
            for (int q = jj - 3; q <= jj; ++q) {
                asm volatile("" : "+v"(k[q]));
                asm volatile("" : "+v"(v[q]));
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// Store L rows of y held as packed words in row-pair mode.
template <int L>
__device__ __forceinline__ void store_pairs(const WaveRows& w, bool valid, const uint32_t (&y)[L / 2]) {
    // lane i < 32 writes row r (its channel and lane 32+i's), lane 32+i writes row r+1
    const uint32_t sel = pair_sel(w.upper);
#pragma unroll
    for (int jj = 0; jj < L / 2; ++jj) {
        const uint32_t word = pair_exchange(y[jj], w.partner, sel);
        if (valid)
            __builtin_amdgcn_raw_buffer_store_b32(word, w.y, w.pair_off, (uint32_t)(2 * jj) * w.row_bytes,
                                                  kStream);
    }
}

// float32 storage (float32 rows, or bfloat16 rows at 2 bytes per lane).  aggregate()
// and weights() replace k by the weights x, which outputs() reuses; y replaces x.
template <typename IO, int L>
struct Chunk {
    static constexpr int kStashRows = 2 * L;
    float k[L], v[L];

    // rows at or beyond nv (wave-uniform) and lanes with !valid read as zero
    __device__ __forceinline__ void load(const WaveRows& w, int nv, bool valid) {
#pragma unroll
        for (int j = 0; j < L; ++j) {
            k[j] = 0.f;
            v[j] = 0.f;
            if (j < nv && valid) {
                k[j] = load_elt<IO>(w.k, w.lane_off, (uint32_t)j * w.row_bytes);
                v[j] = load_elt<IO>(w.v, w.lane_off, (uint32_t)j * w.row_bytes);
            }
        }
    }
    __device__ __forceinline__ void range(float& kmax, float& kmin) const {
        kmax = k[0];
        kmin = k[0];
#pragma unroll
        for (int j = 1; j < L; ++j) {
            kmax = fmaxf(kmax, k[j]);
            kmin = fminf(kmin, k[j]);
        }
    }
    __device__ __forceinline__ Carry aggregate(const Chan& ch, float R) {
        float a = 0.f, b = 0.f;
#pragma unroll
        for (int j = 0; j < L; ++j) {
            const float x = ex2(fmaf(k[j], kLog2e, -R));
            k[j] = x;
            a = fmaf(ch.d, a, x * v[j]);
            b = fmaf(ch.d, b, x);
        }
        return Carry{a, b, (double)R};
    }
    __device__ __forceinline__ void weights(float R) {
#pragma unroll
        for (int j = 0; j < L; ++j) k[j] = ex2(fmaf(k[j], kLog2e, -R));
    }
    // needs the weights: call after aggregate() or weights()
    __device__ __forceinline__ Carry outputs(const Chan& ch, const Carry& c, float R) {
        const float s = ex2((float)(c.p - (double)R));
        float a = c.a * s, b = c.b * s;
#pragma unroll
        for (int j = 0; j < L; ++j) {
            const float x = k[j];
            const float xv = x * v[j];
            k[j] = fmaf(ch.eu, xv, a) * rcp(fmaf(ch.eu, x, b));
            a = fmaf(ch.d, a, xv);
            b = fmaf(ch.d, b, x);
        }
        return Carry{a, b, (double)R};
    }
    __device__ __forceinline__ void prefetch_gate(const WaveRows&, bool) {}
    // outputs() times sigmoid(r): the gate rows are read into v's registers once v is spent
    __device__ __forceinline__ Carry outputs_gated(const Chan& ch, const Carry& c, float R, const WaveRows& w,
                                                   bool valid) {
        const Carry out = outputs(ch, c, R);
#pragma unroll
        for (int j = 0; j < L; ++j) v[j] = valid ? load_elt<IO>(w.r, w.lane_off, (uint32_t)j * w.row_bytes) : 0.f;
#pragma unroll
        for (int j = 0; j < L; ++j) k[j] *= sigmoid_f(v[j]);
        return out;
    }
    __device__ __forceinline__ void store(const WaveRows& w, bool valid) const {
#pragma unroll
        for (int j = 0; j < L; ++j)
            if (valid) store_elt<IO>(w.y, w.lane_off, (uint32_t)j * w.row_bytes, k[j]);
    }
    __device__ __forceinline__ void stash(uint32_t (*st)[64], int lane) const {
#pragma unroll
        for (int j = 0; j < L; ++j) {
            st[j][lane] = __float_as_uint(k[j]);
            st[L + j][lane] = __float_as_uint(v[j]);
        }
    }
    __device__ __forceinline__ void unstash(const uint32_t (*st)[64], int lane) {
#pragma unroll
        for (int j = 0; j < L; ++j) {
            k[j] = __uint_as_float(st[j][lane]);
            v[j] = __uint_as_float(st[L + j][lane]);
        }
    }
};

// Opaque copy of a register: the compiler may not assume the value unchanged, so it
// cannot keep values derived from the register earlier alive to reuse them later.
__device__ __forceinline__ void reg_fence(uint32_t& x) { asm("" : "+v"(x)); }

// bfloat16 row pairs, kept packed: word j holds tokens 2j (low half) and 2j+1 (high
// half) of this lane's channel, so L tokens of k and v take L VGPRs.  The weights are
// recomputed by outputs() (bit for bit the values aggregate() used); y replaces k,
// packed the same way (rounded to nearest even once, from float32).  Every phase
// unpacks again behind reg_fence(): otherwise the compiler keeps all 2L unpacked
// floats alive between phases, which doubles the registers of a chunk.
template <int L>
struct Chunk<Bf16Pair, L> {
    static_assert(L % 2 == 0, "tokens come in row pairs");
    static constexpr int kStashRows = L;
    uint32_t k[L / 2], v[L / 2];

    __device__ __forceinline__ void fence() {
#pragma unroll
        for (int jj = 0; jj < L / 2; ++jj) {
            reg_fence(k[jj]);
            reg_fence(v[jj]);
        }
    }

    __device__ __forceinline__ void load(const WaveRows& w, int nv, bool valid) { load_pairs<L>(w, nv, valid, k, v); }
    __device__ __forceinline__ void range(float& kmax, float& kmin) const {
        kmax = bf_lo(k[0]);
        kmin = kmax;
#pragma unroll
        for (int jj = 0; jj < L / 2; ++jj) {
            const float k0 = bf_lo(k[jj]), k1 = bf_hi(k[jj]);
            kmax = fmaxf(kmax, fmaxf(k0, k1));
            kmin = fminf(kmin, fminf(k0, k1));
        }
    }
    __device__ __forceinline__ Carry aggregate(const Chan& ch, float R) {
        fence();
        float a = 0.f, b = 0.f;
#pragma unroll
        for (int jj = 0; jj < L / 2; ++jj) {
            const float x0 = ex2(fmaf(bf_lo(k[jj]), kLog2e, -R));
            a = fmaf(ch.d, a, x0 * bf_lo(v[jj]));
            b = fmaf(ch.d, b, x0);
            const float x1 = ex2(fmaf(bf_hi(k[jj]), kLog2e, -R));
            a = fmaf(ch.d, a, x1 * bf_hi(v[jj]));
            b = fmaf(ch.d, b, x1);
        }
        return Carry{a, b, (double)R};
    }
    __device__ __forceinline__ void weights(float) {}
    __device__ __forceinline__ Carry outputs(const Chan& ch, const Carry& c, float R) {
        fence();
        const float s = ex2((float)(c.p - (double)R));
        float a = c.a * s, b = c.b * s;
#pragma unroll
        for (int jj = 0; jj < L / 2; ++jj) {
            float y[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const float kf = h ? bf_hi(k[jj]) : bf_lo(k[jj]);
                const float vf = h ? bf_hi(v[jj]) : bf_lo(v[jj]);
                const float x = ex2(fmaf(kf, kLog2e, -R));
                const float xv = x * vf;
                y[h] = fmaf(ch.eu, xv, a) * rcp(fmaf(ch.eu, x, b));
                a = fmaf(ch.d, a, xv);
                b = fmaf(ch.d, b, x);
            }
            k[jj] = pack_bf16(y[0], y[1]);
        }
        return Carry{a, b, (double)R};
    }
    // outputs() times sigmoid(r), rounded to bf16 once: the float32 outputs of pair jj stay
    // unpacked in k[jj] and v[jj] (both spent once the pair is done) until they meet their gate.
    // The gate's row-pair words of the first kGateAhead pairs are loaded by prefetch_gate()
    // into registers of their own, before the tile's look-back; once pair jj is gated and
    // packed, v[jj] is free and takes the gate word of pair jj + kGateAhead.
    static constexpr int kGateAhead = 16;
    uint32_t gate_ahead[kGateAhead];
    __device__ __forceinline__ void prefetch_gate(const WaveRows& w, bool valid) {
#pragma unroll
        for (int jj = 0; jj < kGateAhead; ++jj)
            gate_ahead[jj] = valid ? __builtin_amdgcn_raw_buffer_load_b32(w.r, w.pair_off,
                                                                          (uint32_t)(2 * jj) * w.row_bytes, kStream)
                                   : 0u;
    }
    __device__ __forceinline__ Carry outputs_gated(const Chan& ch, const Carry& c, float R, const WaveRows& w,
                                                   bool valid) {
        fence();
        const float s = ex2((float)(c.p - (double)R));
        float a = c.a * s, b = c.b * s;
#pragma unroll
        for (int jj = 0; jj < L / 2; ++jj) {
            float y[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const float kf = h ? bf_hi(k[jj]) : bf_lo(k[jj]);
                const float vf = h ? bf_hi(v[jj]) : bf_lo(v[jj]);
                const float x = ex2(fmaf(kf, kLog2e, -R));
                const float xv = x * vf;
                y[h] = fmaf(ch.eu, xv, a) * rcp(fmaf(ch.eu, x, b));
                a = fmaf(ch.d, a, xv);
                b = fmaf(ch.d, b, x);
            }
            k[jj] = __float_as_uint(y[0]);
            v[jj] = __float_as_uint(y[1]);
        }
        const uint32_t sel = pair_sel(w.upper);
#pragma unroll
        for (int jj = 0; jj < L / 2; ++jj) {
            const uint32_t gw = jj < kGateAhead ? gate_ahead[jj] : v[jj - kGateAhead];
            const uint32_t rw = pair_exchange(gw, w.partner, sel);
            k[jj] = pack_bf16(__uint_as_float(k[jj]) * sigmoid_f(bf_lo(rw)),
                              __uint_as_float(v[jj]) * sigmoid_f(bf_hi(rw)));
            if (jj + kGateAhead < L / 2) {
                // the load's offset is tied to the packed pair, so the compiler cannot hoist the
                // load above it (and hold every gate word at once)
                uint32_t voff = w.pair_off;
                asm volatile("" : "+v"(voff) : "v"(k[jj]));
                v[jj] = valid ? __builtin_amdgcn_raw_buffer_load_b32(
                                    w.r, voff, (uint32_t)(2 * (jj + kGateAhead)) * w.row_bytes, kStream)
                              : 0u;
            }
        }
        return Carry{a, b, (double)R};
    }
    __device__ __forceinline__ void store(const WaveRows& w, bool valid) const { store_pairs<L>(w, valid, k); }
    __device__ __forceinline__ void stash(uint32_t (*st)[64], int lane) const {
#pragma unroll
        for (int jj = 0; jj < L / 2; ++jj) {
            st[jj][lane] = k[jj];
            st[L / 2 + jj][lane] = v[jj];
        }
    }
    __device__ __forceinline__ void unstash(const uint32_t (*st)[64], int lane) {
#pragma unroll
        for (int jj = 0; jj < L / 2; ++jj) {
            k[jj] = st[jj][lane];
            v[jj] = st[L / 2 + jj][lane];
        }
    }
};

// Tokens per lane per chunk: 32 float32 values of k and v, or 64 packed bfloat16 ones,
// keep a chunk in 64 VGPRs.
template <typename IO>
constexpr int chunk_tokens() { return kPair<IO> ? 64 : 32; }

// ----------------------------------------------------------------------------
// Sequential kernel
// ----------------------------------------------------------------------------

// grid: x covers the channels of one batch row, y is the batch row.  bfloat16 row pairs: a
// wave's 64 channels move as two rows per instruction, as in the chunked kernel (every lane
// of the wave then takes part in the exchanges; lanes past C only skip their loads and stores).
template <typename IO, int L, bool GATE>
__global__ __launch_bounds__(256) void fwd_seq_kernel(FwdArgs args) {
    const int C = args.C, T = args.T;
    const int bi = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int c_grp = blockIdx.x * 256 + (threadIdx.x & ~63);
    const int c = c_grp + (kPair<IO> ? pair_channel(lane) : lane);
    const bool cvalid = c < C;
    if (kPair<IO> ? c_grp >= C : !cvalid) return;  // pairs: only whole waves leave

    const int cw = cvalid ? c : 0;
    const Chan ch = make_chan(args.w[cw], args.u[cw]);
    const size_t si = (size_t)bi * C + cw;
    Carry st = (args.sin_a && cvalid) ? carry_from_abi(args.sin_a[si], args.sin_b[si], args.sin_p[si])
                                      : empty_carry();
    const size_t row_elems = (size_t)bi * T * C + c_grp;

    for (int t0 = 0; t0 < T; t0 += L) {
        const int nv = min(L, T - t0);
        const size_t off = (row_elems + (size_t)t0 * C) * sizeof(IO);
        WaveRows w;
        w.k = make_rsrc(static_cast<const char*>(args.k) + off);
        w.v = make_rsrc(static_cast<const char*>(args.v) + off);
        w.y = make_rsrc(static_cast<char*>(args.y) + off);
        if constexpr (GATE) w.r = make_rsrc(static_cast<const char*>(args.r) + off);
        w.lane_off = (uint32_t)((c - c_grp) * sizeof(IO));
        w.row_bytes = (uint32_t)(C * sizeof(IO));
        w.pair_off = (uint32_t)((lane & 31) * 4) + (uint32_t)(lane >> 5) * w.row_bytes;
        w.upper = (uint32_t)(lane >> 5);
        w.partner = (uint32_t)((lane ^ 32) << 2);
        Chunk<IO, L> chunk;
        chunk.load(w, nv, cvalid);
        float kmax, kmin;
        chunk.range(kmax, kmin);
        st = normalize(st);
        const float R = kmax * kLog2e;
        // the ragged last chunk walks exactly
        const bool ok = nv == L && chunk_fast_ok(ch, kmax, kmin) && (st.p - (double)R <= (double)kSpan);
        if (__all(ok)) {
            chunk.weights(R);
            if constexpr (GATE) {
                if constexpr (kPair<IO>) chunk.prefetch_gate(w, cvalid);
                st = chunk.outputs_gated(ch, st, R, w, cvalid);
            } else {
                st = chunk.outputs(ch, st, R);
            }
            chunk.store(w, cvalid);
        } else {
            lse_walk<IO, true, GATE>(ch, st, w, nv, cvalid, cvalid);
        }
    }
    if (args.sout_a && cvalid) carry_to_abi(st, args.sout_a[si], args.sout_b[si], args.sout_p[si]);
}

// ----------------------------------------------------------------------------
// Chunked single-pass kernel
// ----------------------------------------------------------------------------
//
// Records.  Every tile publishes, per channel, two states: slot 0 the aggregate of
// the tile alone, slot 1 the inclusive state after the tile (float32 form, see
// rec_form).  Each of a, b, p is stored as its own 64-bit word (value | tag << 32)
// with tag = (epoch << 2) | kind; the epoch changes at every launch, so a word belongs
// to this launch exactly when its tag matches.  Words are written and read with
// device-scope atomics (single-copy atomic at 64 bits), so a reader never accepts a
// torn or stale value and no fence or store-drain is needed.  A per-tile status word
// (the strongest kind published) lets a look-back inspect 64 consecutive chunks of a
// group in one contiguous read; it is only a hint: every record word the fold
// consumes is re-validated by its own tag.
//
// Layout: status[g][chunk] (u32), so one look-back read covers 64 consecutive chunks
// of its group, and rec[chunk][g][slot][comp][lane] (u64, comp = a, b, p).  Records are
// chunk-major because the tiles in flight at any moment share a chunk index and have
// consecutive groups: their records then form one dense region instead of landing a
// large power-of-two stride apart, which would pile the traffic onto a few channels.
//
// Launch bookkeeping lives in the workspace's control block and needs no kernel of its
// own: tiles take tickets from a counter; every workgroup counts itself done at its
// end, and the last one resets both counters and advances the epoch for the next
// launch (every other workgroup has read the epoch and taken its ticket by then).

// Aggregate records a look-back loads per round of its forward fold.  Registers for the
// batch are reserved by every wave (the look-back's code path shares the allocation with
// the waves that keep their chunk), so the batch is one record: float32 tiles fold 0.3
// records on average (B=8, T=8192, C=2048) and packed bfloat16 tiles 1.6 (B=1, T=65536,
// C=5120), and a batch of two measured no faster.
template <typename IO>
constexpr int fold_batch() { return 1; }

struct TileRecs {
    uint64_t* rec;       // records of chunk 0 of this group
    uint32_t* status;    // this group's status words
    size_t chunk_words;  // words per chunk index over all groups: n_groups * 6 * 64
    uint32_t tag_agg, tag_incl;
    uint32_t give_up_word;  // value of the give-up word that stops this launch
    __device__ __forceinline__ uint64_t* word(int chunk, int slot, int comp, int lane) const {
        return rec + (size_t)chunk * chunk_words + (size_t)(slot * 3 + comp) * 64 + lane;
    }
};

// Publish the record of `slot` for this lane's channel, then the tile's status hint.
__device__ __forceinline__ void publish(const TileRecs& R, int chunk, int slot, int lane, const Carry& c,
                                        uint32_t tag) {
    st_word(R.word(chunk, slot, 0, lane), c.a, tag);
    st_word(R.word(chunk, slot, 1, lane), c.b, tag);
    st_word(R.word(chunk, slot, 2, lane), (float)c.p, tag);
    if (lane == 0) __hip_atomic_store(&R.status[chunk], tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The float32 form a state takes in a record: float32 reference pf and the exact
// residual factor 2^(p - pf) folded into a and b (same A and B up to one rounding).
__device__ __forceinline__ Carry rec_form(const Carry& c) {
    const float pf = fmaxf((float)c.p, -3.0e38f);
    const float r = ex2((float)(c.p - (double)pf));
    return Carry{c.a * r, c.b * r, (double)pf};
}

// One link of the canonical chain of inclusive states: the state after the previous
// tile (record form) advanced over a tile whose aggregate is `agg` (record form).
// Every tile and every look-back computes inclusive states with exactly this sequence
// of operations, so the bits do not depend on which record a look-back starts from.
__device__ __forceinline__ Carry advance(const Carry& prev, const Carry& agg, double decay) {
    return rec_form(combine(normalize(prev), agg, decay));
}

// The state entering chunk ci (ci >= 1): lane l inspects the status of chunk ci-1-l,
// 64 chunks per window, until the nearest inclusive record is found with every chunk
// after it published; the state is then folded forward from that inclusive record
// through the aggregates in chunk order with advance(), reproducing the canonical
// chain bit for bit.  Gives up (raising the give-up word) after kMaxSpins polls, or
// soon after another tile has given up, so every wave always finishes.
template <int TILE, int FB>
__device__ __forceinline__ bool look_back(const FwdArgs& args, const TileRecs& R, const Chan& ch, int ci,
                                          int lane, Carry& out) {
    // every poll reads the previous chunk's inclusive record, which ends the search at once when
    // complete (one round trip instead of the status word's and then the record's), together
    // with the status words of the 64 chunks before this one
    int start;
    for (uint32_t spin = 0;; ++spin) {
        uint64_t inc[3];
        bool good = true;
#pragma unroll
        for (int q = 0; q < 3; ++q) {
            inc[q] = ld_word(R.word(ci - 1, 1, q, lane));
            good = good && word_tag(inc[q]) == R.tag_incl;
        }
        const int pc = ci - 1 - lane;
        const uint32_t st = pc >= 0 ? ld_status(&R.status[pc]) : 0u;
        if (__all(good)) {
            out = Carry{word_val(inc[0]), word_val(inc[1]), (double)word_val(inc[2])};
            return true;
        }
        start = scan_window<-1>(st, pc >= 0, ci - 1, ci, R.tag_agg, R.tag_incl);
        if (start >= 0) break;
        if (start == kWindowAllReady) {  // 64 aggregates: continue the search beyond the window
            start = find_inclusive<-1>(R.status, args.n_chunks, ci - 64, lane, R.tag_agg, R.tag_incl, args.ctrl,
                                       R.give_up_word);
            if (start < 0) return false;
            break;
        }
        if (must_stop(args.ctrl, R.give_up_word, spin)) return raise_give_up(args.ctrl, R.give_up_word, lane);
        __builtin_amdgcn_s_sleep(kPollSleep);
    }
    // fold forward from the inclusive record of `start` through the aggregates after it,
    // FB aggregates per round; the first round also loads the inclusive record, and a
    // round re-reads its words until every tag matches
    const double decay = (double)TILE * w2_of(ch);
    Carry P{0.f, 0.f, 0.0};
    bool have_p = false;
#pragma unroll 1
    for (int c0 = start + 1;;) {
        const int n = min(FB, ci - c0);
        uint64_t inc[3], t[FB][3];
        for (uint32_t spin = 0;; ++spin) {
            bool good = true;
            if (!have_p)
#pragma unroll
                for (int q = 0; q < 3; ++q) {
                    inc[q] = ld_word(R.word(start, 1, q, lane));
                    good = good && word_tag(inc[q]) == R.tag_incl;
                }
#pragma unroll
            for (int j = 0; j < FB; ++j)
                if (j < n)
#pragma unroll
                    for (int q = 0; q < 3; ++q) {
                        t[j][q] = ld_word(R.word(c0 + j, 0, q, lane));
                        good = good && word_tag(t[j][q]) == R.tag_agg;
                    }
            if (__all(good)) break;
            if (must_stop(args.ctrl, R.give_up_word, spin)) return raise_give_up(args.ctrl, R.give_up_word, lane);
            __builtin_amdgcn_s_sleep(kPollSleep);
        }
        if (!have_p) {
            P = Carry{word_val(inc[0]), word_val(inc[1]), (double)word_val(inc[2])};
            have_p = true;
        }
#pragma unroll
        for (int j = 0; j < FB; ++j)
            if (j < n) P = advance(P, Carry{word_val(t[j][0]), word_val(t[j][1]), (double)word_val(t[j][2])}, decay);
        c0 += n;
        if (c0 >= ci) break;
    }
    out = P;
    return true;
}

// The state entering chunk ci (ci >= 1) without waiting on any other tile, for a tile whose
// look-back gave up or a launch forced onto that path: from the nearest chunk before ci
// whose inclusive record is complete (else the start of the sequence: the state in, or the
// empty state), through every chunk after it, by its aggregate record when that is complete,
// else by walking the chunk's TILE rows of k and v in memory with the exact per-token
// recurrence.  Every record word used is validated by its own tag; nothing is waited for, so
// the result is the state the WKV equation defines whatever the other tiles are doing.
// rows_k, rows_v: this lane's group at time step 0 of its sequence (channel c_grp).
template <typename IO, int TILE>
__device__ __forceinline__ Carry rebuild_prefix(const FwdArgs& args, const TileRecs& R, const Chan& ch, int ci, int lane,
                                             const char* rows_k, const char* rows_v, uint32_t lane_off, bool cvalid,
                                             size_t si) {
    // nearest complete inclusive record, 64 chunks per look, nothing waited for
    int start = -1;
    Carry P{0.f, 0.f, 0.0};
    for (int nearest = ci - 1; nearest >= 0 && start < 0; nearest -= 64) {
        const int pc = nearest - lane;
        const uint32_t st = pc >= 0 ? ld_status(&R.status[pc]) : 0u;
        uint64_t cand = __ballot(pc >= 0 && st == R.tag_incl);
        while (cand) {
            const int d = __builtin_ctzll(cand);
            uint64_t wds[3];
            bool good = true;
#pragma unroll
            for (int q = 0; q < 3; ++q) {
                wds[q] = ld_word(R.word(nearest - d, 1, q, lane));
                good = good && word_tag(wds[q]) == R.tag_incl;
            }
            if (__all(good)) {
                start = nearest - d;
                P = Carry{word_val(wds[0]), word_val(wds[1]), (double)word_val(wds[2])};
                break;
            }
            cand &= cand - 1ull;
        }
    }
    if (start < 0)
        P = rec_form((args.sin_a && cvalid) ? carry_from_abi(args.sin_a[si], args.sin_b[si], args.sin_p[si])
                                             : empty_carry());
    const double decay = (double)TILE * w2_of(ch);
    const uint32_t row_bytes = (uint32_t)((size_t)args.C * sizeof(IO));
#pragma unroll 1
    for (int m = start + 1; m < ci; ++m) {
        uint64_t t[3];
        bool good = true;
#pragma unroll
        for (int q = 0; q < 3; ++q) {
            t[q] = ld_word(R.word(m, 0, q, lane));
            good = good && word_tag(t[q]) == R.tag_agg;
        }
        if (__all(good)) {
            P = advance(P, Carry{word_val(t[0]), word_val(t[1]), (double)word_val(t[2])}, decay);
        } else {
            Carry cw = normalize(P);
            const size_t off = (size_t)m * TILE * row_bytes;
            walk_rows_exact<IO>(ch, cw, rows_k + off, rows_v + off, lane_off, row_bytes, TILE, cvalid);
            P = rec_form(cw);
        }
    }
    return P;
}

// Everything a tile's waves share.
template <int NW, int STASH_ROWS>
struct TileShared {
    int ticket;
    float a[NW][64];  // per-wave aggregate, then the state before each wave
    float b[NW][64];
    double p[NW][64];
    float ca[64];  // state entering the tile
    float cb[64];
    double cp[64];
    uint32_t stash[STASH_ROWS][64];  // wave 0's chunk while it runs the look-back
};

// The tile after its k, v rows are loaded.  FAST: the wave's chunk is full and well
// conditioned and stays in registers; otherwise the wave walks its rows in memory with
// the exact log-sum-exp recurrence.  Both instantiations pass the same two barriers.
template <typename IO, int L, int NW, bool FAST, bool GATE, bool BYIDX>
__device__ __forceinline__ void tile_body(const FwdArgs& args, TileShared<NW, Chunk<IO, L>::kStashRows>& sh,
                                          const TileRecs& recs, const WaveRows& rows, Chunk<IO, L>& chunk,
                                          const Chan& ch, float R, int lane, int wid, int ci, int bi, int c,
                                          bool cvalid, int nv, int t_tile, int tile_len, int g, bool forced,
                                          size_t seq_off) {
    constexpr int TILE = L * NW;
    const int C = args.C, T = args.T;

    // ---- per-wave aggregate of its tokens, from the empty state ----
    Carry agg;
    if constexpr (FAST) {
        agg = chunk.aggregate(ch, R);
    } else {
        agg = empty_carry();
        lse_walk<IO, false>(ch, agg, rows, nv, cvalid, false);
    }
    // the gate's first rows load while the tile waits for its entering state
    if constexpr (FAST && GATE) chunk.prefetch_gate(rows, cvalid);
    sh.a[wid][lane] = agg.a;
    sh.b[wid][lane] = agg.b;
    sh.p[wid][lane] = agg.p;
    __syncthreads();

    // ---- wave 0: tile aggregate, look-back, publish ----
    if (wid == 0) {
        // numbered by index: a ticket past the launch's tiles shows a counter that was not zero
        if (BYIDX && (uint32_t)__builtin_amdgcn_readfirstlane(sh.ticket) >=
                         (uint32_t)args.n_groups * (uint32_t)args.n_chunks) {
            forced = true;
            flag_stale_ticket(args.ctrl);
        }
        // the previous tile's inclusive record, read first: when it is complete, as it usually is
        // by the time the tile has its aggregate, the look-back is skipped
        uint64_t pv[3];
#pragma unroll
        for (int q = 0; q < 3; ++q) pv[q] = ci > 0 ? ld_word(recs.word(ci - 1, 1, q, lane)) : 0ull;
        if constexpr (FAST) {
            chunk.stash(sh.stash, lane);
            // the chunk must really leave the registers: no forwarding of the stash
            asm volatile("" ::: "memory");
        }
        Carry run = empty_carry();
        // unrolled by four: each step's exponents and scale factors overlap the previous step's
        // sums (B=8, T=1024, C=768 float32 at 16 waves: 19.2 -> 18.6 us, the same bits)
#pragma unroll 4
        for (int wv = 0; wv < NW; ++wv) {
            const int nvw = max(0, min(L, T - (t_tile + wv * L)));
            const Carry aw{sh.a[wv][lane], sh.b[wv][lane], sh.p[wv][lane]};
            sh.a[wv][lane] = run.a;  // slot wv now holds the state before wave wv
            sh.b[wv][lane] = run.b;
            sh.p[wv][lane] = run.p;
            run = combine(run, aw, (double)nvw * w2_of(ch));
        }
        const Carry agg_rec = rec_form(run);
        Carry prefix;
        const size_t si = (size_t)bi * C + c;
        if (ci == 0) {
            prefix = rec_form((args.sin_a && cvalid) ? carry_from_abi(args.sin_a[si], args.sin_b[si], args.sin_p[si])
                                                      : empty_carry());
        } else {
            bool ready = !forced;
#pragma unroll
            for (int q = 0; q < 3; ++q) ready = ready && word_tag(pv[q]) == recs.tag_incl;
            bool have = false;
            if (__all(ready)) {
                prefix = Carry{word_val(pv[0]), word_val(pv[1]), (double)word_val(pv[2])};
                have = true;
            } else if (!forced) {
                publish(recs, ci, 0, lane, agg_rec, recs.tag_agg);
                have = look_back<TILE, fold_batch<IO>()>(args, recs, ch, ci, lane, prefix);
            } else {
                raise_give_up(args.ctrl, recs.give_up_word, lane);
            }
            if (!have) {
                prefix = rebuild_prefix<IO, TILE>(args, recs, ch, ci, lane, static_cast<const char*>(args.k) + seq_off,
                                                  static_cast<const char*>(args.v) + seq_off, rows.lane_off, cvalid, si);
            }
        }
        const Carry incl = advance(prefix, agg_rec, (double)tile_len * w2_of(ch));
        if (ci + 1 < args.n_chunks) {
            publish(recs, ci, 1, lane, incl, recs.tag_incl);
        } else if (args.sout_a && cvalid) {
            carry_to_abi(incl, args.sout_a[si], args.sout_b[si], args.sout_p[si]);
        }
        sh.ca[lane] = prefix.a;
        sh.cb[lane] = prefix.b;
        sh.cp[lane] = prefix.p;
        if constexpr (FAST) {
            asm volatile("" ::: "memory");
            chunk.unstash(sh.stash, lane);
        }
    }
    __syncthreads();
    if (nv == 0) return;

    // ---- outputs of this wave from the state entering its tokens ----
    const Carry tile_in{sh.ca[lane], sh.cb[lane], sh.cp[lane]};
    const Carry before{sh.a[wid][lane], sh.b[wid][lane], sh.p[wid][lane]};
    const Carry cin = normalize(combine(tile_in, before, (double)(wid * L) * w2_of(ch)));
    if (args.dump_a) {
        // the state entering every kBwdTile-th time step, for the backward scan
        const int t0 = t_tile + wid * L;
        if (t0 % kBwdTile == 0) {
            const Carry r = rec_form(cin);
            const size_t di = ((size_t)(t0 / kBwdTile) * args.n_groups + g) * 64 + (c & 63);
            args.dump_a[di] = r.a;
            args.dump_b[di] = r.b;
            args.dump_p[di] = (float)r.p;
        }
        if (args.y == nullptr) return;  // no y: the states were all that was asked
    }
    if (FAST && __all(cin.p - (double)R <= (double)kSpan)) {
        if constexpr (GATE)
            chunk.outputs_gated(ch, cin, R, rows, cvalid);
        else
            chunk.outputs(ch, cin, R);
        chunk.store(rows, cvalid);
    } else {
        Carry c2 = cin;
        lse_walk<IO, true, GATE>(ch, c2, rows, nv, cvalid, cvalid);
    }
}

template <typename IO, int L, int NW, bool GATE, bool BYIDX>
__global__ __launch_bounds__(64 * NW, NW >= 2 ? 4 : 1) void fwd_chunked_kernel(FwdArgs args) {
    constexpr int TILE = L * NW;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform (scalar) index
    const int C = args.C, T = args.T;
    __shared__ TileShared<NW, Chunk<IO, L>::kStashRows> sh;

    // Tiles are numbered in the order workgroups start, so every tile this one waits on
    // has already started and publishes its aggregate without waiting for anything.  When
    // every tile of the launch can be resident at once, the workgroup index numbers them
    // instead and the loads start without waiting for a ticket (all tiles then run
    // together, and the ticket, taken after the loads, only checks the counter).
    const uint32_t n_tiles = (uint32_t)args.n_groups * (uint32_t)args.n_chunks;
    bool forced = false;
    int ticket;
    if constexpr (BYIDX) {
        ticket = (int)blockIdx.x;
    } else {
        if (threadIdx.x == 0) sh.ticket = (int)atomicAdd(&args.ctrl[kCtrlTicket], 1u);
        __syncthreads();
        ticket = (int)remap_ticket((uint32_t)__builtin_amdgcn_readfirstlane(sh.ticket), n_tiles, args.ctrl, forced);
    }
    const int g = ticket % args.n_groups;
    const int ci = ticket / args.n_groups;
    const int bi = g / args.groups_per_row;
    const int c_grp = (g - bi * args.groups_per_row) * 64;
    const int c = c_grp + (kPair<IO> ? pair_channel(lane) : lane);
    const bool cvalid = c < C;
    const int t_tile = ci * TILE;
    const int t0 = __builtin_amdgcn_readfirstlane(t_tile + wid * L);
    const int nv = max(0, min(L, T - t0));
    const int tile_len = min(TILE, T - t_tile);

    WaveRows rows;
    {
        const size_t off = (((size_t)bi * T + (size_t)min(t0, T)) * C + c_grp) * sizeof(IO);
        rows.k = make_rsrc(static_cast<const char*>(args.k) + off);
        rows.v = make_rsrc(static_cast<const char*>(args.v) + off);
        rows.y = make_rsrc(static_cast<char*>(args.y) + off);
        if constexpr (GATE) rows.r = make_rsrc(static_cast<const char*>(args.r) + off);
        rows.lane_off = (uint32_t)((c - c_grp) * sizeof(IO));
        rows.row_bytes = (uint32_t)(C * sizeof(IO));
        rows.pair_off = (uint32_t)((lane & 31) * 4) + (uint32_t)(lane >> 5) * rows.row_bytes;
        rows.upper = (uint32_t)(lane >> 5);
        rows.partner = (uint32_t)((lane ^ 32) << 2);
    }
    Chunk<IO, L> chunk;
    chunk.load(rows, nv, cvalid);
    if (BYIDX && threadIdx.x == 0) sh.ticket = (int)atomicAdd(&args.ctrl[kCtrlTicket], 1u);

    // read after the loads are issued; constant during the launch
    const uint32_t epoch = __builtin_amdgcn_readfirstlane(args.ctrl[kCtrlEpoch]);
    forced = forced || launch_forced(args.ctrl);
    TileRecs recs;
    recs.rec = static_cast<uint64_t*>(args.recs) + (size_t)g * 6 * 64;
    recs.chunk_words = (size_t)args.n_groups * 6 * 64;
    recs.status = args.status + (size_t)g * args.n_chunks;
    recs.tag_agg = (epoch << 2) | kKindAgg;
    recs.tag_incl = (epoch << 2) | kKindIncl;
    recs.give_up_word = epoch | kCtrlGiveUpMark;

    const int cw = cvalid ? c : 0;
    const Chan ch = make_chan(args.w[cw], args.u[cw]);
    float kmax, kmin;
    chunk.range(kmax, kmin);
    const float R = kmax * kLog2e;
    // the fast path takes full chunks only; the one ragged chunk at the end of a
    // sequence (and any ill-conditioned chunk) walks its rows exactly
    const size_t seq_off = ((size_t)bi * T * C + c_grp) * sizeof(IO);  // time step 0 of this group
    if (__all(chunk_fast_ok(ch, kmax, kmin)) && nv == L)
        tile_body<IO, L, NW, true, GATE, BYIDX>(args, sh, recs, rows, chunk, ch, R, lane, wid, ci, bi, c, cvalid, nv,
                                         t_tile, tile_len, g, forced, seq_off);
    else
        tile_body<IO, L, NW, false, GATE, BYIDX>(args, sh, recs, rows, chunk, ch, R, lane, wid, ci, bi, c, cvalid, nv,
                                          t_tile, tile_len, g, forced, seq_off);

    // ---- launch bookkeeping: the last workgroup to finish prepares the next launch ----
    __syncthreads();
    if (threadIdx.x == 0) finish_tile(args.ctrl, n_tiles, epoch, false);
}

// One control word of a workspace set from the stream (no memset: callers may capture it).
__global__ void set_word_kernel(uint32_t* __restrict__ p, uint32_t value) {
    if (threadIdx.x == 0) __hip_atomic_store(p, value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

hipError_t launch_set_word(uint32_t* p, uint32_t value, hipStream_t s) {
    hipLaunchKernelGGL(set_word_kernel, dim3(1), dim3(64), 0, s, p, value);
    return hipGetLastError();
}

// Zero a workspace (the state every workspace must start from).
__global__ void zero_words_kernel(uint32_t* __restrict__ p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

// State copy used when T = 0 and the caller asked for the state through.
__global__ void copy_state_kernel(const float* __restrict__ ia, const float* __restrict__ ib,
                                  const float* __restrict__ ip, float* __restrict__ oa, float* __restrict__ ob,
                                  float* __restrict__ op, long n) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    oa[i] = ia ? ia[i] : 0.f;
    ob[i] = ib ? ib[i] : 0.f;
    op[i] = ip ? ip[i] : kEmptyPf;
}

// ----------------------------------------------------------------------------
// Launchers
// ----------------------------------------------------------------------------

template <typename IO>
static hipError_t launch_seq_t(const FwdArgs& a, hipStream_t s) {
    constexpr int L = 32;  // tokens per chunk (bf16 row pairs: 16 packed words of k and of v)
    const long blocks = (a.C + 255) / 256;
    if (a.r)
        hipLaunchKernelGGL((fwd_seq_kernel<IO, L, true>), dim3((unsigned)blocks, (unsigned)a.B), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((fwd_seq_kernel<IO, L, false>), dim3((unsigned)blocks, (unsigned)a.B), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_fwd_seq(const FwdArgs& a, int io, hipStream_t s) {
    switch (io) {
        case kIoF32: return launch_seq_t<float>(a, s);
        case kIoBf16: return launch_seq_t<uint16_t>(a, s);
        case kIoBf16Pair: return launch_seq_t<Bf16Pair>(a, s);
    }
    return hipErrorInvalidValue;
}

template <typename IO, int NW, bool BYIDX>
static void launch_chunked_g(const FwdArgs& a, hipStream_t s) {
    constexpr int L = chunk_tokens<IO>();
    const long n_tiles = (long)a.n_groups * a.n_chunks;
    if (a.r)
        hipLaunchKernelGGL((fwd_chunked_kernel<IO, L, NW, true, BYIDX>), dim3((unsigned)n_tiles), dim3(64 * NW), 0, s,
                           a);
    else
        hipLaunchKernelGGL((fwd_chunked_kernel<IO, L, NW, false, BYIDX>), dim3((unsigned)n_tiles), dim3(64 * NW), 0,
                           s, a);
}

template <typename IO, int NW>
static hipError_t launch_chunked_t(const FwdArgs& a, hipStream_t s) {
    if (a.by_index)
        launch_chunked_g<IO, NW, true>(a, s);
    else
        launch_chunked_g<IO, NW, false>(a, s);
    return hipGetLastError();
}

// Workgroups of the index-numbered kernel that one compute unit holds at once (0 if unknown),
// looked up once per instantiation.
template <typename IO, int NW>
static int resident_t(bool gate) {
    constexpr int L = chunk_tokens<IO>();
    static std::atomic<int> cached[2];
    int n = cached[gate].load(std::memory_order_relaxed);
    if (n > 0) return n;
    hipError_t e = gate ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fwd_chunked_kernel<IO, L, NW, true, true>,
                                                                       64 * NW, 0)
                        : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fwd_chunked_kernel<IO, L, NW, false, true>,
                                                                       64 * NW, 0);
    if (e != hipSuccess || n <= 0) return 0;
    cached[gate].store(n, std::memory_order_relaxed);
    return n;
}

template <typename IO>
static int resident_n(int tile, bool gate) {
    constexpr int L = chunk_tokens<IO>();
    if constexpr (L == 64) {
        switch (tile) {
            case 64: return resident_t<IO, 1>(gate);
            case 128: return resident_t<IO, 2>(gate);
            case 256: return resident_t<IO, 4>(gate);
            case 512: return resident_t<IO, 8>(gate);
        }
    } else {
        switch (tile) {
            case 64: return resident_t<IO, 2>(gate);
            case 128: return resident_t<IO, 4>(gate);
            case 256: return resident_t<IO, 8>(gate);
            case 512: return resident_t<IO, 16>(gate);
        }
    }
    return 0;
}

int fwd_chunked_resident_per_cu(int io, int tile, bool gate) {
    switch (io) {
        case kIoF32: return resident_n<float>(tile, gate);
        case kIoBf16: return resident_n<uint16_t>(tile, gate);
        case kIoBf16Pair: return resident_n<Bf16Pair>(tile, gate);
    }
    return 0;
}

// Tile = NW waves x chunk_tokens tokens, 64 channels; at most 16 waves (1024 threads).
template <typename IO>
static hipError_t launch_chunked_n(const FwdArgs& a, int tile, hipStream_t s) {
    constexpr int L = chunk_tokens<IO>();
    if constexpr (L == 64) {
        switch (tile) {
            case 64: return launch_chunked_t<IO, 1>(a, s);
            case 128: return launch_chunked_t<IO, 2>(a, s);
            case 256: return launch_chunked_t<IO, 4>(a, s);
            case 512: return launch_chunked_t<IO, 8>(a, s);
        }
    } else {
        switch (tile) {
            case 64: return launch_chunked_t<IO, 2>(a, s);
            case 128: return launch_chunked_t<IO, 4>(a, s);
            case 256: return launch_chunked_t<IO, 8>(a, s);
            case 512: return launch_chunked_t<IO, 16>(a, s);
        }
    }
    return hipErrorInvalidValue;
}

hipError_t launch_fwd_chunked(const FwdArgs& a, int io, int tile, hipStream_t s) {
    switch (io) {
        case kIoF32: return launch_chunked_n<float>(a, tile, s);
        case kIoBf16: return launch_chunked_n<uint16_t>(a, tile, s);
        case kIoBf16Pair: return launch_chunked_n<Bf16Pair>(a, tile, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_zero_words(void* p, size_t n_words, hipStream_t s) {
    const size_t blocks = std::min<size_t>(4096, (n_words + 255) / 256 + 1);
    hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<uint32_t*>(p),
                       n_words);
    return hipGetLastError();
}

hipError_t launch_copy_state(const float* ia, const float* ib, const float* ip, float* oa, float* ob, float* op,
                             long n, hipStream_t s) {
    hipLaunchKernelGGL(copy_state_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, ia, ib, ip, oa, ob,
                       op, n);
    return hipGetLastError();
}

}  // namespace wkv
