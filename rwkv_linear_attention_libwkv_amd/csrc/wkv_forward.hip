// Whole-sequence WKV forward kernels for gfx950.
//
// Operator: page "Reinventing RNNs for the Transformer Era: RWKV" (velog review),
// section "WKV 연산자" (WKV equation) and section "RNN-유사추론" (RNN form).  The
// page's time-parallel training mode (section "Transformer-유사학습") runs every
// other op over batch and time at once and only WKV "as a scan"; the two kernels
// here are that scan.
//
// Layout: k, v, y are [B, T, C] with C fastest.  A thread owns NCH consecutive
// channels of one batch row, so a wavefront reads 64*NCH contiguous channels of
// one time step per load (1 KiB for fp32 with NCH=4).
//
//  * fwd_seq_kernel: each thread walks all T for its channels, L tokens at a time
//    (the chunk fast path of wkv_device.h with a per-chunk reference).
//  * fwd_chunked_kernel: single pass over HBM.  A workgroup of NW waves owns one
//    tile = (64*NCH channels) x (NW*L tokens); every wave keeps its L tokens of k, v
//    in registers, reduces them to a per-wave state, the waves are combined in LDS
//    into the tile's aggregate, and the tile's incoming state is obtained from the
//    tiles before it by a decoupled look-back over published per-tile states (the
//    chained-scan technique of Merrill and Garland, "Single-pass Parallel Prefix
//    Scan with Decoupled Look-back", 2016).  Each wave then produces its outputs
//    from its registers, so k and v are read once and y written once.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "wkv_device.h"
#include "wkv_kernels.h"

namespace wkv {

// ----------------------------------------------------------------------------
// Row loads and stores: NCH consecutive channels of one time step.
//
// A wave addresses its rows through a buffer resource whose base is wave-uniform
// (scalar registers), a per-lane 32-bit byte offset (one VGPR for all rows) and a
// per-row scalar offset, so a chunk of rows costs no per-row address registers.
// ----------------------------------------------------------------------------

typedef __amdgpu_buffer_rsrc_t Rsrc;
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ Rsrc make_rsrc(const void* base) {
    // raw buffer (stride 0), 2^31-1 addressable bytes, gfx9 data-format word
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
}

__device__ __forceinline__ float bf_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

template <typename IO, int NCH>
__device__ __forceinline__ void load_row(Rsrc r, uint32_t voff, uint32_t soff, float (&o)[NCH]) {
    if constexpr (sizeof(IO) == 4) {
        if constexpr (NCH == 4) {
            const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
            o[0] = __uint_as_float(t.x); o[1] = __uint_as_float(t.y);
            o[2] = __uint_as_float(t.z); o[3] = __uint_as_float(t.w);
        } else if constexpr (NCH == 2) {
            const u32x2 t = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
            o[0] = __uint_as_float(t.x); o[1] = __uint_as_float(t.y);
        } else {
            o[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
        }
    } else {
        if constexpr (NCH == 4) {
            const u32x2 t = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
            o[0] = bf_lo(t.x); o[1] = bf_hi(t.x); o[2] = bf_lo(t.y); o[3] = bf_hi(t.y);
        } else if constexpr (NCH == 2) {
            const uint32_t t = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
            o[0] = bf_lo(t); o[1] = bf_hi(t);
        } else {
            o[0] = bf_lo((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0));
        }
    }
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// float32 pair -> packed bfloat16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    f32x2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

template <typename IO, int NCH>
__device__ __forceinline__ void store_row(Rsrc r, uint32_t voff, uint32_t soff, const float (&o)[NCH]) {
    if constexpr (sizeof(IO) == 4) {
        if constexpr (NCH == 4) {
            const u32x4 t = {__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]),
                             __float_as_uint(o[3])};
            __builtin_amdgcn_raw_buffer_store_b128(t, r, voff, soff, 0);
        } else if constexpr (NCH == 2) {
            const u32x2 t = {__float_as_uint(o[0]), __float_as_uint(o[1])};
            __builtin_amdgcn_raw_buffer_store_b64(t, r, voff, soff, 0);
        } else {
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o[0]), r, voff, soff, 0);
        }
    } else {
        if constexpr (NCH == 4) {
            const u32x2 t = {pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3])};
            __builtin_amdgcn_raw_buffer_store_b64(t, r, voff, soff, 0);
        } else if constexpr (NCH == 2) {
            __builtin_amdgcn_raw_buffer_store_b32(pack_bf16(o[0], o[1]), r, voff, soff, 0);
        } else {
            __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(pack_bf16(o[0], 0.f) & 0xffffu), r,
                                                  voff, soff, 0);
        }
    }
}

// The rows of one wave: k, v, y resources based at the wave's first row and first channel.
struct WaveRows {
    Rsrc k, v, y;
    uint32_t lane_off;   // byte offset of this lane's first channel
    uint32_t row_bytes;  // C * sizeof(IO)
};

// ----------------------------------------------------------------------------
// Per-chunk arithmetic.
// ----------------------------------------------------------------------------

// Fast path over the tokens of one chunk held in registers, from carry c (normalised)
// with reference R: overwrites xy[j] = 2^(k_j log2e - R) with y_j and returns the state
// after the chunk.
template <int L, bool RAGGED>
__device__ __forceinline__ Carry fast_outputs(const Chan& ch, const Carry& c, float R,
                                              float (&xy)[L], const float (&v)[L], int nv) {
    const float s = ex2((float)(c.p - (double)R));
    float a = c.a * s, b = c.b * s;
#pragma unroll
    for (int j = 0; j < L; ++j) {
        if (RAGGED && j >= nv) break;
        const float x = xy[j];
        const float xv = x * v[j];
        const float ex = ch.eu * x;
        const float num = fmaf(ex, v[j], a);
        const float den = b + ex;
        xy[j] = num * rcp(den);
        a = fmaf(ch.d, a, xv);
        b = fmaf(ch.d, b, x);
    }
    return Carry{a, b, (double)R};
}

// One token of the exact log-sum-exp recurrence (any input, including huge exponent
// ranges, negative w, Inf and NaN).  Returns y when OUT; advances c.
template <bool OUT>
__device__ __forceinline__ float lse_token(const Chan& ch, Carry& c, float k, float v) {
    const double k2 = (double)k * kLog2eD;
    float y = 0.f;
    if (OUT) {
        const double uk = u2_of(ch) + k2;
        const double q = fmax(c.p, uk);
        const float e1 = ex2((float)(c.p - q));
        const float e2 = ex2((float)(uk - q));
        y = fmaf(e1, c.a, e2 * v) * rcp(fmaf(e1, c.b, e2));
    }
    const double pw = c.p - w2_of(ch);
    const double q2 = fmax(pw, k2);
    const float f1 = ex2((float)(pw - q2));
    const float f2 = ex2((float)(k2 - q2));
    c.a = fmaf(f1, c.a, f2 * v);
    c.b = fmaf(f1, c.b, f2);
    c.p = q2;
    return y;
}

// Fallback walk over n tokens read from memory (rows t0 .. t0+n-1 at stride C), advancing
// the NCH carries; writes y rows when yp is non-null.  Rolled loop: this path is rare and
// keeps no chunk in registers.
// Fallback walk over the wave's first n rows, advancing the NCH carries; writes y rows
// when OUT and `store`.  Rolled loop: this path is rare and keeps no chunk in registers.
template <typename IO, int NCH, bool OUT>
__device__ __forceinline__ void lse_walk(const Chan (&ch)[NCH], Carry (&c)[NCH], const WaveRows& w,
                                         int n, bool load, bool store) {
#pragma unroll 1
    for (int j = 0; j < n; ++j) {
        float kr[NCH], vr[NCH], yr[NCH];
        const uint32_t so = (uint32_t)j * w.row_bytes;
        if (load) {
            load_row<IO, NCH>(w.k, w.lane_off, so, kr);
            load_row<IO, NCH>(w.v, w.lane_off, so, vr);
        } else {
#pragma unroll
            for (int i = 0; i < NCH; ++i) { kr[i] = 0.f; vr[i] = 0.f; }
        }
#pragma unroll
        for (int i = 0; i < NCH; ++i) yr[i] = lse_token<OUT>(ch[i], c[i], kr[i], vr[i]);
        if (OUT && store) store_row<IO, NCH>(w.y, w.lane_off, so, yr);
    }
}

// Overwrite a register chunk with zeros (ends the live range of what it held).
template <int NCH, int L>
__device__ __forceinline__ void drop_chunk(float (&kk)[NCH][L], float (&vv)[NCH][L]) {
#pragma unroll
    for (int i = 0; i < NCH; ++i)
#pragma unroll
        for (int j = 0; j < L; ++j) { kk[i][j] = 0.f; vv[i][j] = 0.f; }
}

// max and min of k over the valid tokens
template <int L, bool RAGGED>
__device__ __forceinline__ void k_range(const float (&k)[L], int nv, float& kmax, float& kmin) {
    kmax = k[0];
    kmin = k[0];
#pragma unroll
    for (int j = 1; j < L; ++j) {
        if (RAGGED && j >= nv) break;
        kmax = fmaxf(kmax, k[j]);
        kmin = fminf(kmin, k[j]);
    }
}

// Load the wave's first L rows of NCH channels; rows at or beyond nv (wave-uniform) and
// lanes with !valid read as zero.
template <typename IO, int NCH, int L>
__device__ __forceinline__ void load_chunk(const WaveRows& w, int nv, bool valid,
                                           float (&kk)[NCH][L], float (&vv)[NCH][L]) {
#pragma unroll
    for (int j = 0; j < L; ++j) {
        float kr[NCH], vr[NCH];
#pragma unroll
        for (int i = 0; i < NCH; ++i) { kr[i] = 0.f; vr[i] = 0.f; }
        if (j < nv && valid) {
            load_row<IO, NCH>(w.k, w.lane_off, (uint32_t)j * w.row_bytes, kr);
            load_row<IO, NCH>(w.v, w.lane_off, (uint32_t)j * w.row_bytes, vr);
        }
#pragma unroll
        for (int i = 0; i < NCH; ++i) { kk[i][j] = kr[i]; vv[i][j] = vr[i]; }
    }
}

template <typename IO, int NCH, int L>
__device__ __forceinline__ void store_chunk(const WaveRows& w, int nv, const float (&yy)[NCH][L]) {
#pragma unroll
    for (int j = 0; j < L; ++j) {
        if (j < nv) {
            float yr[NCH];
#pragma unroll
            for (int i = 0; i < NCH; ++i) yr[i] = yy[i][j];
            store_row<IO, NCH>(w.y, w.lane_off, (uint32_t)j * w.row_bytes, yr);
        }
    }
}

// ----------------------------------------------------------------------------
// Sequential kernel
// ----------------------------------------------------------------------------

// grid: x covers the channels of one batch row (NCH per thread), y is the batch row.
template <typename IO, int NCH, int L>
__global__ __launch_bounds__(256) void fwd_seq_kernel(FwdArgs args) {
    const int C = args.C, T = args.T;
    const int bi = blockIdx.y;
    const int c = (blockIdx.x * 256 + threadIdx.x) * NCH;
    if (c >= C) return;

    Chan ch[NCH];
    Carry st[NCH];
    bool chan_ok = true;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        ch[i] = make_chan(args.w[c + i], args.u[c + i]);
        chan_ok = chan_ok && chan_fast_ok(ch[i]);
        const size_t si = (size_t)bi * C + c + i;
        st[i] = args.sin_a ? carry_from_abi(args.sin_a[si], args.sin_b[si], args.sin_p[si])
                           : empty_carry();
    }
    const size_t row_elems = (size_t)bi * T * C;
    const uint32_t row_bytes = (uint32_t)(C * sizeof(IO));

    for (int t0 = 0; t0 < T; t0 += L) {
        const int nv = min(L, T - t0);
        const size_t off = (row_elems + (size_t)t0 * C) * sizeof(IO);
        WaveRows w;
        w.k = make_rsrc(static_cast<const char*>(args.k) + off);
        w.v = make_rsrc(static_cast<const char*>(args.v) + off);
        w.y = make_rsrc(static_cast<char*>(args.y) + off);
        w.lane_off = (uint32_t)(c * sizeof(IO));
        w.row_bytes = row_bytes;
        float kk[NCH][L], vv[NCH][L];
        load_chunk<IO, NCH, L>(w, nv, true, kk, vv);
        float R[NCH];
        bool ok = chan_ok && nv == L;  // the ragged last chunk walks exactly
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            float kmax, kmin;
            k_range<L, false>(kk[i], L, kmax, kmin);
            st[i] = normalize(st[i]);
            R[i] = kmax * kLog2e;
            const float range = (kmax - kmin) * kLog2e;
            ok = ok && (range <= kSpan) && (range - ch[i].u * kLog2e <= kSpan) &&
                 (st[i].p - (double)R[i] <= (double)kSpan);
        }
        if (__all(ok)) {
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
#pragma unroll
                for (int j = 0; j < L; ++j) kk[i][j] = ex2(fmaf(kk[i][j], kLog2e, -R[i]));
                st[i] = fast_outputs<L, false>(ch[i], st[i], R[i], kk[i], vv[i], L);
            }
            store_chunk<IO, NCH, L>(w, L, kk);
        } else {
            lse_walk<IO, NCH, true>(ch, st, w, nv, true, true);
        }
    }
    if (args.sout_a) {
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const size_t si = (size_t)bi * C + c + i;
            float a, b, p;
            carry_to_abi(st[i], a, b, p);
            args.sout_a[si] = a;
            args.sout_b[si] = b;
            args.sout_p[si] = p;
        }
    }
}

// ----------------------------------------------------------------------------
// Chunked single-pass kernel
// ----------------------------------------------------------------------------
//
// Records.  Every tile publishes, per channel, two states: slot 0 the aggregate of
// the tile alone, slot 1 the inclusive state after the tile (float32 form, see
// rec_form).  Each of a, b, p is stored as its own 64-bit word (value | tag << 32)
// with tag = (epoch << 2) | kind; the epoch is bumped by the prep kernel at every
// launch, so a word belongs to this launch exactly when its tag matches.  Words are
// written and read with device-scope atomics (single-copy atomic at 64 bits), so a
// reader never accepts a torn or stale value and no fence or store-drain is needed.
// A per-tile status word (the strongest kind published) lets a look-back inspect 64
// consecutive chunks of a group in one contiguous read; it is only a hint: every
// record word the fold consumes is re-validated by its own tag.
//
// Layout: status[g][chunk] (u32), so one look-back read covers 64 consecutive chunks
// of its group, and rec[chunk][g][slot][comp][col] (u64, comp = a, b, p).  Records are
// chunk-major because the tiles in flight at any moment share a chunk index and have
// consecutive groups: their records then form one dense region instead of landing a
// large power-of-two stride apart, which would pile the traffic onto a few channels.

constexpr uint32_t kKindAgg = 1u;
constexpr uint32_t kKindIncl = 2u;
constexpr uint32_t kMaxSpins = 1u << 18;
constexpr int kFoldBatch = 4;  // aggregate records loaded per round of the forward fold
constexpr int kPollSleep = 2;  // s_sleep between polls (units of 64 clocks)

struct TileRecs {
    uint64_t* rec;     // records of chunk 0 of this group
    uint32_t* status;  // this group's status words
    int GW;
    size_t chunk_words;  // words per chunk index over all groups: n_groups * 6 * GW
    uint32_t tag_agg, tag_incl;
    __device__ __forceinline__ uint64_t* word(int chunk, int slot, int comp, int col) const {
        return rec + (size_t)chunk * chunk_words + (size_t)(slot * 3 + comp) * GW + col;
    }
};

__device__ __forceinline__ void st_word(uint64_t* p, float v, uint32_t tag) {
    __hip_atomic_store(p, ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_word(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t word_tag(uint64_t w) { return (uint32_t)(w >> 32); }
__device__ __forceinline__ float word_val(uint64_t w) { return __uint_as_float((uint32_t)w); }

// Publish the record of `slot` for this lane's channels, then the tile's status hint.
template <int NCH>
__device__ __forceinline__ void publish(const TileRecs& R, int chunk, int slot, int lane,
                                        const Carry (&c)[NCH], uint32_t tag) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int col = lane * NCH + i;
        st_word(R.word(chunk, slot, 0, col), c[i].a, tag);
        st_word(R.word(chunk, slot, 1, col), c[i].b, tag);
        st_word(R.word(chunk, slot, 2, col), (float)c[i].p, tag);
    }
    if (lane == 0)
        __hip_atomic_store(&R.status[chunk], tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// Raise the give-up flag (once per wave) and report failure.
__device__ __forceinline__ bool give_up(const FwdArgs& args, int lane) {
    if (lane == 0) atomicOr(&args.ctrl[kCtrlGiveUp], 1u);
    return false;
}

__device__ __forceinline__ bool gave_up_elsewhere(const FwdArgs& args) {
    return __hip_atomic_load(&args.ctrl[kCtrlGiveUp], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
}

__device__ __forceinline__ bool should_stop(const FwdArgs& args, uint32_t spin) {
    return spin >= kMaxSpins || ((spin & 31u) == 31u && gave_up_elsewhere(args));
}

// Read the record of (chunk, slot) for this lane's channels, re-reading until every
// word carries `tag`.  Returns false after giving up.
template <int NCH>
__device__ __forceinline__ bool read_record(const FwdArgs& args, const TileRecs& R, int chunk, int slot,
                                            uint32_t tag, int lane, Carry (&out)[NCH]) {
    for (uint32_t spin = 0;; ++spin) {
        bool good = true;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int col = lane * NCH + i;
            const uint64_t a = ld_word(R.word(chunk, slot, 0, col));
            const uint64_t b = ld_word(R.word(chunk, slot, 1, col));
            const uint64_t p = ld_word(R.word(chunk, slot, 2, col));
            good = good && word_tag(a) == tag && word_tag(b) == tag && word_tag(p) == tag;
            out[i] = Carry{word_val(a), word_val(b), (double)word_val(p)};
        }
        if (__all(good)) return true;
        if (should_stop(args, spin)) return give_up(args, lane);
        __builtin_amdgcn_s_sleep(kPollSleep);
    }
}

// Look-back for tile (chunk ci): the state entering the tile.  Lane l reads the status
// of the chunk l+1 back until the nearest inclusive record is found with every chunk
// after it published; the state is then folded forward from that inclusive record
// through the aggregates in chunk order with advance(), reproducing the canonical chain
// bit for bit.  Gives up (raising the give-up flag) after kMaxSpins polls, or soon after another
// tile has given up, so every wave always finishes.
template <int NCH, int TILE>
__device__ __forceinline__ bool look_back(const FwdArgs& args, const TileRecs& R, const Chan (&ch)[NCH],
                                          int ci, int lane, Carry (&out)[NCH]) {
    int nearest = ci - 1;  // chunk inspected by lane 0 in the current window
    int start = -1;        // chunk holding the nearest inclusive record
    for (;;) {
        const int pc = nearest - lane;
        const int nlanes = min(64, nearest + 1);
        bool window_done = false;
        for (uint32_t spin = 0;; ++spin) {
            const uint32_t st = pc >= 0 ? __hip_atomic_load(&R.status[pc], __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT)
                                        : 0u;
            const bool is_incl = pc >= 0 && st == R.tag_incl;
            const bool is_ready = is_incl || (pc >= 0 && st == R.tag_agg);
            const uint64_t incl = __ballot(is_incl);
            const uint64_t ready = __ballot(is_ready);
            if (incl) {
                const int d = __builtin_ctzll(incl);
                const uint64_t need = (d >= 63) ? ~0ull : ((2ull << d) - 1ull);
                if ((ready & need) == need) { start = nearest - d; break; }
            } else if (nlanes == 64 && ready == ~0ull) {
                window_done = true;  // 64 aggregates, no inclusive record yet: look further back
                break;
            }
            if (should_stop(args, spin)) return give_up(args, lane);
            __builtin_amdgcn_s_sleep(kPollSleep);
        }
        if (!window_done) break;
        nearest -= 64;
    }
    Carry P[NCH];
    if (!read_record<NCH>(args, R, start, 1, R.tag_incl, lane, P)) return false;
    double decay[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) decay[i] = (double)TILE * w2_of(ch[i]);
    // forward fold over the aggregates, kFoldBatch records per round; a round re-reads
    // its batch until every word's tag matches
#pragma unroll 1
    for (int c0 = start + 1; c0 < ci; c0 += kFoldBatch) {
        const int n = min(kFoldBatch, ci - c0);
        uint64_t t[kFoldBatch][NCH][3];
        for (uint32_t spin = 0;; ++spin) {
            bool good = true;
#pragma unroll
            for (int j = 0; j < kFoldBatch; ++j)
                if (j < n)
#pragma unroll
                    for (int i = 0; i < NCH; ++i)
#pragma unroll
                        for (int q = 0; q < 3; ++q) {
                            t[j][i][q] = ld_word(R.word(c0 + j, 0, q, lane * NCH + i));
                            good = good && word_tag(t[j][i][q]) == R.tag_agg;
                        }
            if (__all(good)) break;
            if (should_stop(args, spin)) return give_up(args, lane);
            __builtin_amdgcn_s_sleep(kPollSleep);
        }
#pragma unroll
        for (int j = 0; j < kFoldBatch; ++j)
            if (j < n)
#pragma unroll
                for (int i = 0; i < NCH; ++i)
                    P[i] = advance(P[i],
                                   Carry{word_val(t[j][i][0]), word_val(t[j][i][1]),
                                         (double)word_val(t[j][i][2])},
                                   decay[i]);
    }
#pragma unroll
    for (int i = 0; i < NCH; ++i) out[i] = P[i];
    return true;
}

// Everything a tile's waves share.
template <int NCH, int L, int NW>
struct TileShared {
    int ticket;
    float a[NW][64 * NCH];  // per-wave aggregate, then the state before each wave
    float b[NW][64 * NCH];
    double p[NW][64 * NCH];
    float ca[64 * NCH];  // state entering the tile
    float cb[64 * NCH];
    double cp[64 * NCH];
    float stash[2 * NCH * L][64];  // wave 0's chunk while it runs the look-back
};

// The tile after its k, v rows are loaded.  FAST: the wave's chunk is full and well
// conditioned and stays in registers; otherwise the wave walks its rows in memory with
// the exact log-sum-exp recurrence.  Both instantiations pass the same two barriers.
template <typename IO, int NCH, int L, int NW, bool FAST>
__device__ __forceinline__ void tile_body(const FwdArgs& args, TileShared<NCH, L, NW>& sh,
                                          const TileRecs& recs, const WaveRows& rows,
                                          float (&kk)[NCH][L], float (&vv)[NCH][L],
                                          const Chan (&ch)[NCH], const float (&R)[NCH], int lane,
                                          int wid, int g, int ci, int bi, int c, bool cvalid, int nv,
                                          int t_tile, int tile_len) {
    constexpr int TILE = L * NW;
    const int C = args.C, T = args.T;

    // ---- per-wave aggregate of its tokens, from the empty state ----
    Carry agg[NCH];
    if constexpr (FAST) {
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            float a = 0.f, b = 0.f;
#pragma unroll
            for (int j = 0; j < L; ++j) {
                const float x = ex2(fmaf(kk[i][j], kLog2e, -R[i]));
                kk[i][j] = x;  // k is replaced by its weight relative to R
                a = fmaf(ch[i].d, a, x * vv[i][j]);
                b = fmaf(ch[i].d, b, x);
            }
            agg[i] = Carry{a, b, (double)R[i]};
        }
    } else {
#pragma unroll
        for (int i = 0; i < NCH; ++i) agg[i] = empty_carry();
        lse_walk<IO, NCH, false>(ch, agg, rows, nv, cvalid, false);
    }
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        sh.a[wid][lane * NCH + i] = agg[i].a;
        sh.b[wid][lane * NCH + i] = agg[i].b;
        sh.p[wid][lane * NCH + i] = agg[i].p;
    }
    __syncthreads();

    // ---- wave 0: tile aggregate, look-back, publish ----
    if (wid == 0) {
        if constexpr (FAST) {
#pragma unroll
            for (int i = 0; i < NCH; ++i)
#pragma unroll
                for (int j = 0; j < L; ++j) {
                    sh.stash[i * L + j][lane] = kk[i][j];
                    sh.stash[(NCH + i) * L + j][lane] = vv[i][j];
                }
            // the chunk must really leave the registers: no forwarding of the stash
            asm volatile("" ::: "memory");
        }
        Carry run[NCH];
#pragma unroll
        for (int i = 0; i < NCH; ++i) run[i] = empty_carry();
#pragma unroll 1
        for (int wv = 0; wv < NW; ++wv) {
            const int nvw = max(0, min(L, T - (t_tile + wv * L)));
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                const int col = lane * NCH + i;
                const Carry aw{sh.a[wv][col], sh.b[wv][col], sh.p[wv][col]};
                sh.a[wv][col] = run[i].a;  // slot wv now holds the state before wave wv
                sh.b[wv][col] = run[i].b;
                sh.p[wv][col] = run[i].p;
                run[i] = combine(run[i], aw, (double)nvw * w2_of(ch[i]));
            }
        }
        Carry agg_rec[NCH];
#pragma unroll
        for (int i = 0; i < NCH; ++i) agg_rec[i] = rec_form(run[i]);
        Carry prefix[NCH];
        if (ci == 0) {
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                const size_t si = (size_t)bi * C + c + i;
                prefix[i] = rec_form((args.sin_a && cvalid)
                                         ? carry_from_abi(args.sin_a[si], args.sin_b[si], args.sin_p[si])
                                         : empty_carry());
            }
        } else {
            publish<NCH>(recs, ci, 0, lane, agg_rec, recs.tag_agg);
            if (!look_back<NCH, TILE>(args, recs, ch, ci, lane, prefix)) {
#pragma unroll
                for (int i = 0; i < NCH; ++i) prefix[i] = empty_carry();
            }
        }
        Carry incl[NCH];
#pragma unroll
        for (int i = 0; i < NCH; ++i)
            incl[i] = advance(prefix[i], agg_rec[i], (double)tile_len * w2_of(ch[i]));
        if (ci + 1 < args.n_chunks) {
            publish<NCH>(recs, ci, 1, lane, incl, recs.tag_incl);
        } else if (args.sout_a && cvalid) {
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                const size_t si = (size_t)bi * C + c + i;
                float a, b, p;
                carry_to_abi(incl[i], a, b, p);
                args.sout_a[si] = a;
                args.sout_b[si] = b;
                args.sout_p[si] = p;
            }
        }
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            sh.ca[lane * NCH + i] = prefix[i].a;
            sh.cb[lane * NCH + i] = prefix[i].b;
            sh.cp[lane * NCH + i] = prefix[i].p;
        }
        if constexpr (FAST) {
            asm volatile("" ::: "memory");
#pragma unroll
            for (int i = 0; i < NCH; ++i)
#pragma unroll
                for (int j = 0; j < L; ++j) {
                    kk[i][j] = sh.stash[i * L + j][lane];
                    vv[i][j] = sh.stash[(NCH + i) * L + j][lane];
                }
        }
    }
    __syncthreads();
    if (nv == 0) return;

    // ---- outputs of this wave from the state entering its tokens ----
    Carry cin[NCH];
    bool out_ok = FAST;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int col = lane * NCH + i;
        const Carry tile_in{sh.ca[col], sh.cb[col], sh.cp[col]};
        const Carry before{sh.a[wid][col], sh.b[wid][col], sh.p[wid][col]};
        cin[i] = normalize(combine(tile_in, before, (double)(wid * L) * w2_of(ch[i])));
        out_ok = out_ok && (cin[i].p - (double)R[i] <= (double)kSpan);
    }
    if (FAST && __all(out_ok)) {
#pragma unroll
        for (int i = 0; i < NCH; ++i) fast_outputs<L, false>(ch[i], cin[i], R[i], kk[i], vv[i], L);
        if (cvalid) store_chunk<IO, NCH, L>(rows, L, kk);
    } else {
        lse_walk<IO, NCH, true>(ch, cin, rows, nv, cvalid, cvalid);
    }
}

template <typename IO, int NCH, int L, int NW>
__global__ __launch_bounds__(64 * NW) void fwd_chunked_kernel(FwdArgs args) {
    constexpr int GW = 64 * NCH;
    constexpr int TILE = L * NW;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform (scalar) index
    const int C = args.C, T = args.T;
    __shared__ TileShared<NCH, L, NW> sh;

    // Tiles are numbered in the order workgroups start, so every tile this one waits on
    // has already started and publishes its aggregate without waiting for anything.
    if (threadIdx.x == 0) sh.ticket = (int)atomicAdd(&args.ctrl[kCtrlTicket], 1u);
    __syncthreads();
    const int ticket = __builtin_amdgcn_readfirstlane(sh.ticket);
    const uint32_t epoch = __builtin_amdgcn_readfirstlane(args.ctrl[kCtrlEpoch]);
    const int g = ticket % args.n_groups;
    const int ci = ticket / args.n_groups;
    const int bi = g / args.groups_per_row;
    const int c_grp = (g - bi * args.groups_per_row) * GW;
    const int c = c_grp + lane * NCH;
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
        rows.lane_off = (uint32_t)(lane * NCH * sizeof(IO));
        rows.row_bytes = (uint32_t)(C * sizeof(IO));
    }
    TileRecs recs;
    recs.rec = static_cast<uint64_t*>(args.recs) + (size_t)g * 6 * GW;
    recs.chunk_words = (size_t)args.n_groups * 6 * GW;
    recs.status = args.status + (size_t)g * args.n_chunks;
    recs.GW = GW;
    recs.tag_agg = (epoch << 2) | kKindAgg;
    recs.tag_incl = (epoch << 2) | kKindIncl;

    float kk[NCH][L], vv[NCH][L];
    load_chunk<IO, NCH, L>(rows, nv, cvalid, kk, vv);

    Chan ch[NCH];
    bool ok = true;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int ci_ = cvalid ? c + i : 0;
        ch[i] = Chan{args.chan_d[ci_], args.chan_eu[ci_], args.w[ci_], args.u[ci_]};
        ok = ok && chan_fast_ok(ch[i]);
    }
    float R[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        float kmax, kmin;
        k_range<L, false>(kk[i], L, kmax, kmin);
        R[i] = kmax * kLog2e;
        const float range = (kmax - kmin) * kLog2e;
        ok = ok && (range <= kSpan) && (range - ch[i].u * kLog2e <= kSpan);
    }
    // the fast path takes full chunks only; the one ragged chunk at the end of a
    // sequence (and any ill-conditioned chunk) walks its rows exactly
    if (__all(ok) && nv == L)
        tile_body<IO, NCH, L, NW, true>(args, sh, recs, rows, kk, vv, ch, R, lane, wid, g, ci, bi, c,
                                        cvalid, nv, t_tile, tile_len);
    else
        tile_body<IO, NCH, L, NW, false>(args, sh, recs, rows, kk, vv, ch, R, lane, wid, g, ci, bi, c,
                                         cvalid, nv, t_tile, tile_len);
}

// Per launch: reset the ticket counter and give-up flag, open a new record epoch, and
// compute the per-channel constants e^{-w} and e^{u} once (float64 exp, rounded).
__global__ void prep_kernel(uint32_t* __restrict__ ctrl, const float* __restrict__ w,
                            const float* __restrict__ u, float* __restrict__ cd,
                            float* __restrict__ ceu, int C) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i == 0) {
        ctrl[kCtrlTicket] = 0u;
        ctrl[kCtrlGiveUp] = 0u;
        ctrl[kCtrlEpoch] = (ctrl[kCtrlEpoch] + 1u) & 0x3fffffffu;
    }
    if (i < C) {
        cd[i] = (float)exp(-(double)w[i]);
        ceu[i] = (float)exp((double)u[i]);
    }
}

// Zero a workspace (the state every workspace must start from).
__global__ void zero_words_kernel(uint32_t* __restrict__ p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

// State copy used when T = 0 and the caller asked for the state through.
__global__ void copy_state_kernel(const float* __restrict__ ia, const float* __restrict__ ib,
                                  const float* __restrict__ ip, float* __restrict__ oa,
                                  float* __restrict__ ob, float* __restrict__ op, long n) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    oa[i] = ia ? ia[i] : 0.f;
    ob[i] = ib ? ib[i] : 0.f;
    op[i] = ip ? ip[i] : kEmptyPf;
}

// ----------------------------------------------------------------------------
// Launchers
// ----------------------------------------------------------------------------

// Tokens per thread per chunk: NCH * L = 32 keeps k and v of a chunk in 64 VGPRs.
template <int NCH>
constexpr int chunk_tokens() { return 32 / NCH; }

template <typename IO, int NCH>
static hipError_t launch_seq_t(const FwdArgs& a, hipStream_t s) {
    constexpr int L = chunk_tokens<NCH>();
    const long per_row = a.C / NCH;
    const long blocks = (per_row + 255) / 256;
    hipLaunchKernelGGL((fwd_seq_kernel<IO, NCH, L>), dim3((unsigned)blocks, (unsigned)a.B), dim3(256),
                       0, s, a);
    return hipGetLastError();
}

// Channels per thread: only NCH = 1 is instantiated at present (wider rows raise the
// register count past four waves per SIMD).
hipError_t launch_fwd_seq(const FwdArgs& a, int dtype, int nch, hipStream_t s) {
    if (nch != 1) return hipErrorInvalidValue;
    return dtype == 0 ? launch_seq_t<float, 1>(a, s) : launch_seq_t<uint16_t, 1>(a, s);
}

template <typename IO, int NCH, int NW>
static hipError_t launch_chunked_t(const FwdArgs& a, hipStream_t s) {
    constexpr int L = chunk_tokens<NCH>();
    const long n_tiles = (long)a.n_groups * a.n_chunks;
    hipLaunchKernelGGL(prep_kernel, dim3((unsigned)((a.C + 255) / 256)), dim3(256), 0, s, a.ctrl, a.w,
                       a.u, a.chan_d, a.chan_eu, a.C);
    hipLaunchKernelGGL((fwd_chunked_kernel<IO, NCH, L, NW>), dim3((unsigned)n_tiles), dim3(64 * NW),
                       0, s, a);
    return hipGetLastError();
}

// Tile = NW waves x (32 / NCH) tokens.
template <typename IO>
static hipError_t launch_chunked_n(const FwdArgs& a, int nch, int tile, hipStream_t s) {
    if (nch == 2) {
        if (tile == 64) return launch_chunked_t<IO, 2, 4>(a, s);
        if (tile == 128) return launch_chunked_t<IO, 2, 8>(a, s);
        if (tile == 256) return launch_chunked_t<IO, 2, 16>(a, s);
    } else if (nch == 1) {
        if (tile == 64) return launch_chunked_t<IO, 1, 2>(a, s);
        if (tile == 128) return launch_chunked_t<IO, 1, 4>(a, s);
        if (tile == 256) return launch_chunked_t<IO, 1, 8>(a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_fwd_chunked(const FwdArgs& a, int dtype, int nch, int tile, hipStream_t s) {
    return dtype == 0 ? launch_chunked_n<float>(a, nch, tile, s) : launch_chunked_n<uint16_t>(a, nch, tile, s);
}

hipError_t launch_zero_words(void* p, size_t n_words, hipStream_t s) {
    const size_t blocks = std::min<size_t>(4096, (n_words + 255) / 256 + 1);
    hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<uint32_t*>(p), n_words);
    return hipGetLastError();
}

hipError_t launch_copy_state(const float* ia, const float* ib, const float* ip, float* oa,
                             float* ob, float* op, long n, hipStream_t s) {
    hipLaunchKernelGGL(copy_state_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, ia, ib,
                       ip, oa, ob, op, n);
    return hipGetLastError();
}

}  // namespace wkv
