// Backward of the WKV operator for gfx950: gradients of L = sum(gy * y) with respect to
// k, v (per element) and w, u (per (b, c) lane).
//
// Page "Reinventing RNNs for the Transformer Era: RWKV" (velog review), section
// "WKV 연산자" (WKV equation); the time-parallel training mode (section
// "Transformer-유사학습") backpropagates through it.  With alpha_{t,i} the normalised
// weight of token i in y_t, q_t = gy_t / D_t (D_t the WKV denominator) and the reverse
// sums over the later outputs
//   G_i = sum_{t>i} q_t e^{-(t-1-i) w},       H_i = sum_{t>i} q_t y_t e^{-(t-1-i) w},
//   G'_i = sum_{t>i} (t-1-i) q_t e^{-(t-1-i) w},  H'_i likewise with q_t y_t,
// the gradients are
//   dL/dv_i = e^{k_i} G_i + e^{u+k_i} q_i
//   dL/dk_i = e^{k_i} (v_i G_i - H_i) + e^{u+k_i} q_i (v_i - y_i)
//   dL/du   = sum_i e^{u+k_i} q_i (v_i - y_i)
//   dL/dw   = -sum_i e^{k_i} (v_i G'_i - H'_i)
// and the sums obey G_{i-1} = q_i + e^{-w} G_i, H_{i-1} = q_i y_i + e^{-w} H_i,
// G'_{i-1} = e^{-w} (G'_i + G_i), H'_{i-1} = e^{-w} (H'_i + H_i): a scan backwards in time.
//
// Plan (tiles of kBwdTile tokens x 64 channels, aligned with the forward tiles):
//   1. the chunked forward kernel dumps the forward state entering every tile;
//   2. bwd_scan_kernel, a single-pass chained scan backwards in time: per tile, recompute
//      y and q from the dumped state, reduce the tile to its reverse aggregate (the G, H,
//      G', H' it contributes before its start), take the reverse carry entering from the
//      right from the next tile's inclusive record when it has already arrived, else
//      publish the aggregate and find the carry by decoupled look-back over the later
//      tiles, publish the inclusive carry, then walk the tokens backwards writing dL/dk,
//      dL/dv and the tile's dL/dw, dL/du partial sums;
//   3. bwd_reduce_kernel: per lane, sum the partials in a fixed order.
// Every result is a deterministic function of the inputs (the carries follow one
// canonical chain of operations whichever record a look-back starts from, and no sum
// uses atomics), so gradients are bitwise reproducible.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wkv_chain.h"
#include "wkv_device.h"
#include "wkv_kernels.h"
#include "wkv_rows.h"

namespace wkv {

// Reverse sums at one position: G = g 2^r, H = h 2^r, G' = gp 2^r, H' = hp 2^r
// (r a float64 exponent in log2 units).
struct Rev {
    float g, h, gp, hp;
    double r;
};

__device__ __forceinline__ Rev empty_rev() { return {0.f, 0.f, 0.f, 0.f, kEmptyP}; }

// X (an earlier segment of n tokens, its sums at the position before it) followed by
// the carry C (sums at X's last position from the tokens after X): the sums at the
// position before X.  The later tokens are n steps further away, so C decays by
// e^{-n w} and G' gains n G (each distance t-1-i grows by n).
__device__ __forceinline__ Rev fold_rev(const Rev& x, const Rev& c, int n, double w2) {
    const double rc = c.r - (double)n * w2;
    const double rm = fmax(x.r, rc);
    const float fx = ex2((float)(x.r - rm));
    const float fc = ex2((float)(rc - rm));
    const float nf = (float)n;
    return {fmaf(x.g, fx, c.g * fc), fmaf(x.h, fx, c.h * fc), fmaf(x.gp, fx, fmaf(nf, c.g, c.gp) * fc),
            fmaf(x.hp, fx, fmaf(nf, c.h, c.hp) * fc), rm};
}

// Same sums with the largest magnitude scaled into [0.5, 1) by an exact power of two.
__device__ __forceinline__ Rev normalize_rev(const Rev& c) {
    const float m = fmaxf(fmaxf(fabsf(c.g), fabsf(c.h)), fmaxf(fabsf(c.gp), fabsf(c.hp)));
    if (m == 0.f) return empty_rev();
    if (!(m < 3.0e38f)) return c;  // Inf and NaN pass through
    int e;
    (void)__builtin_frexpf(m, &e);
    return {__builtin_ldexpf(c.g, -e), __builtin_ldexpf(c.h, -e), __builtin_ldexpf(c.gp, -e),
            __builtin_ldexpf(c.hp, -e), c.r + (double)e};
}

// The float32 form a carry takes in a record: float32 reference rf and the exact
// residual factor 2^(r - rf) folded into the sums (the same values up to one rounding).
__device__ __forceinline__ Rev rev_rec_form(const Rev& c) {
    const float rf = fmaxf((float)c.r, -3.0e38f);
    const float f = ex2((float)(c.r - (double)rf));
    return {c.g * f, c.h * f, c.gp * f, c.hp * f, (double)rf};
}

// One link of the canonical chain of inclusive carries: the carry entering the later
// tile (record form) folded through a tile of n tokens whose aggregate is `agg` (record
// form).  Tiles and look-backs compute inclusive carries with exactly these operations.
__device__ __forceinline__ Rev advance_rev(const Rev& later, const Rev& agg, int n, double w2) {
    return rev_rec_form(fold_rev(agg, normalize_rev(later), n, w2));
}

// Fast path of one wave's L tokens in the frame of reference R (log2 units): x_j =
// 2^(k_j log2e - R), q^_j = gy_j / (D_j 2^-R), so that every product e^{k_i} q_t of the
// gradients is x_i q^_t.  After forward(): k holds x, g holds q^, y holds y.
template <int L>
struct BwdChunk {
    float k[L], v[L], g[L], y[L];

    // rows at or beyond nv (wave-uniform) and lanes with !valid read as zero
    template <typename IO>
    __device__ __forceinline__ void load(const WaveRows& w, Rsrc gy, int nv, bool valid) {
        if constexpr (kPair<IO>) {
            // row pairs: every 4-byte load first, then the exchanges with the partner lane
            // (all 64 lanes take part in those; only the loads are predicated)
            uint32_t xk[L / 2], xv[L / 2], xg[L / 2];
#pragma unroll
            for (int jj = 0; jj < L / 2; ++jj) {
                xk[jj] = 0u;
                xv[jj] = 0u;
                xg[jj] = 0u;
                if (valid && 2 * jj + (int)w.upper < nv) {
                    const uint32_t so = (uint32_t)(2 * jj) * w.row_bytes;
                    xk[jj] = __builtin_amdgcn_raw_buffer_load_b32(w.k, w.pair_off, so, kStream);
                    xv[jj] = __builtin_amdgcn_raw_buffer_load_b32(w.v, w.pair_off, so, kStream);
                    xg[jj] = __builtin_amdgcn_raw_buffer_load_b32(gy, w.pair_off, so, kStream);
                }
            }
            const uint32_t sel = pair_sel(w.upper);
#pragma unroll
            for (int jj = 0; jj < L / 2; ++jj) {
                const uint32_t pk = pair_exchange(xk[jj], w.partner, sel);
                const uint32_t pv = pair_exchange(xv[jj], w.partner, sel);
                const uint32_t pg = pair_exchange(xg[jj], w.partner, sel);
                k[2 * jj] = bf_lo(pk);
                k[2 * jj + 1] = bf_hi(pk);
                v[2 * jj] = bf_lo(pv);
                v[2 * jj + 1] = bf_hi(pv);
                g[2 * jj] = bf_lo(pg);
                g[2 * jj + 1] = bf_hi(pg);
            }
        } else {
#pragma unroll
            for (int j = 0; j < L; ++j) {
                k[j] = 0.f;
                v[j] = 0.f;
                g[j] = 0.f;
                if (j < nv && valid) {
                    const uint32_t so = (uint32_t)j * w.row_bytes;
                    k[j] = load_elt<IO>(w.k, w.lane_off, so);
                    v[j] = load_elt<IO>(w.v, w.lane_off, so);
                    g[j] = load_elt<IO>(gy, w.lane_off, so);
                }
            }
        }
    }
    // dL/dk (in k) and dL/dv (in v) of a full chunk, after backward()
    template <typename IO>
    __device__ __forceinline__ void store_grads(const WaveRows& w, Rsrc gk, Rsrc gv, bool valid) const {
        store_rows<IO>(w, gk, valid, k);
        store_rows<IO>(w, gv, valid, v);
    }
    // one array of L rows (full chunk), stored in the mode's row format
    template <typename IO>
    static __device__ __forceinline__ void store_rows(const WaveRows& w, Rsrc dst, bool valid, const float (&x)[L]) {
        if constexpr (kPair<IO>) {
            const uint32_t sel = pair_sel(w.upper);
#pragma unroll
            for (int jj = 0; jj < L / 2; ++jj) {
                const uint32_t word = pair_exchange(pack_bf16(x[2 * jj], x[2 * jj + 1]), w.partner, sel);
                if (valid)
                    __builtin_amdgcn_raw_buffer_store_b32(word, dst, w.pair_off, (uint32_t)(2 * jj) * w.row_bytes,
                                                          kStream);
            }
        } else if (valid) {
#pragma unroll
            for (int j = 0; j < L; ++j) store_elt<IO>(dst, w.lane_off, (uint32_t)j * w.row_bytes, x[j]);
        }
    }
    // one array of L rows (full chunk), loaded in the mode's row format
    template <typename IO>
    static __device__ __forceinline__ void load_rows(const WaveRows& w, Rsrc src, bool valid, float (&x)[L]) {
        if constexpr (kPair<IO>) {
            uint32_t xw[L / 2];
#pragma unroll
            for (int jj = 0; jj < L / 2; ++jj)
                xw[jj] = valid ? __builtin_amdgcn_raw_buffer_load_b32(src, w.pair_off, (uint32_t)(2 * jj) * w.row_bytes,
                                                                      kStream)
                               : 0u;
            const uint32_t sel = pair_sel(w.upper);
#pragma unroll
            for (int jj = 0; jj < L / 2; ++jj) {
                const uint32_t p = pair_exchange(xw[jj], w.partner, sel);
                x[2 * jj] = bf_lo(p);
                x[2 * jj + 1] = bf_hi(p);
            }
        } else {
#pragma unroll
            for (int j = 0; j < L; ++j) x[j] = valid ? load_elt<IO>(src, w.lane_off, (uint32_t)j * w.row_bytes) : 0.f;
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
    // forward state of the wave's tokens from the empty state (frame R); k becomes x
    __device__ __forceinline__ Carry aggregate(const Chan& ch, float R) {
        float a = 0.f, b = 0.f;
#pragma unroll
        for (int j = 0; j < L; ++j) {
            k[j] = ex2(fmaf(k[j], kLog2e, -R));
            a = fmaf(ch.d, a, k[j] * v[j]);
            b = fmaf(ch.d, b, k[j]);
        }
        return Carry{a, b, (double)R};
    }
    // y and q^ from the forward state entering the wave (normalised, p - R <= kSpan)
    __device__ __forceinline__ void forward(const Chan& ch, const Carry& cin, float R) {
        const float s = ex2((float)(cin.p - (double)R));
        float a = cin.a * s, b = cin.b * s;
#pragma unroll
        for (int j = 0; j < L; ++j) {
            const float x = k[j];
            const float xv = x * v[j];
            const float inv = rcp(fmaf(ch.eu, x, b));
            y[j] = fmaf(ch.eu, xv, a) * inv;
            g[j] = g[j] * inv;
            a = fmaf(ch.d, a, xv);
            b = fmaf(ch.d, b, x);
        }
    }
    // forward() with the output gate z = sigmoid(r) y: g holds dL/dz on entry and becomes
    // q^ of dL/dy = dL/dz sigmoid(r); r (in sr) is replaced by dL/dr = dL/dy y sigmoid(-r)
    __device__ __forceinline__ void forward_gated(const Chan& ch, const Carry& cin, float R, float (&sr)[L]) {
        const float s = ex2((float)(cin.p - (double)R));
        float a = cin.a * s, b = cin.b * s;
#pragma unroll
        for (int j = 0; j < L; ++j) {
            const float x = k[j];
            const float xv = x * v[j];
            const float inv = rcp(fmaf(ch.eu, x, b));
            y[j] = fmaf(ch.eu, xv, a) * inv;
            const float gyj = g[j] * sigmoid_f(sr[j]);
            sr[j] = gyj * y[j] * sigmoid_f(-sr[j]);
            g[j] = gyj * inv;
            a = fmaf(ch.d, a, xv);
            b = fmaf(ch.d, b, x);
        }
    }
    // reverse sums at the position before the wave from its own tokens (frame R)
    __device__ __forceinline__ Rev reverse_aggregate(const Chan& ch, float R) const {
        float G = 0.f, H = 0.f, Gp = 0.f, Hp = 0.f;
#pragma unroll
        for (int j = L - 1; j >= 0; --j) {
            Gp = ch.d * (Gp + G);
            Hp = ch.d * (Hp + H);
            G = fmaf(ch.d, G, g[j]);
            H = fmaf(ch.d, H, g[j] * y[j]);
        }
        return Rev{G, H, Gp, Hp, -(double)R};
    }
    // wave 0 parks its chunk in LDS while it runs the look-back (keeps registers free)
    __device__ __forceinline__ void stash(float (*st)[64], int lane) const {
#pragma unroll
        for (int j = 0; j < L; ++j) {
            st[j][lane] = k[j];
            st[L + j][lane] = v[j];
            st[2 * L + j][lane] = g[j];
            st[3 * L + j][lane] = y[j];
        }
    }
    __device__ __forceinline__ void unstash(float (*st)[64], int lane) {
#pragma unroll
        for (int j = 0; j < L; ++j) {
            k[j] = st[j][lane];
            v[j] = st[L + j][lane];
            g[j] = st[2 * L + j][lane];
            y[j] = st[3 * L + j][lane];
        }
    }
    // gradients from the reverse carry at the wave's last position; k, v are replaced
    // by dL/dk, dL/dv; accumulates the lane's dL/dw, dL/du
    __device__ __forceinline__ void backward(const Chan& ch, const Rev& cin, float R, float& gw, float& gu) {
        const float s = ex2((float)(cin.r + (double)R));
        float G = cin.g * s, H = cin.h * s, Gp = cin.gp * s, Hp = cin.hp * s;
#pragma unroll
        for (int j = L - 1; j >= 0; --j) {
            const float x = k[j], vj = v[j], qj = g[j], yj = y[j];
            const float cur = ch.eu * x * qj;  // e^{u+k_j} q_j
            const float dvy = vj - yj;
            v[j] = fmaf(x, G, cur);                   // dL/dv_j
            k[j] = fmaf(x, fmaf(vj, G, -H), cur * dvy);  // dL/dk_j
            gw = fmaf(-x, fmaf(vj, Gp, -Hp), gw);
            gu = fmaf(cur, dvy, gu);
            Gp = ch.d * (Gp + G);
            Hp = ch.d * (Hp + H);
            G = fmaf(ch.d, G, qj);
            H = fmaf(ch.d, H, qj * yj);
        }
    }
};

// Exact path for one wave (any input): per token, the forward state is recomputed from
// the state entering the wave by walking the earlier tokens of the wave again (O(L^2),
// read from memory, no per-token arrays), and the reverse sums carry their own float64
// exponent.  Produces the wave's reverse aggregate (pass 0) or its gradients (pass 1);
// with the gate, pass 0 also writes dL/dr unless WRITE_GR is off (a tile rebuilding
// another tile's carry writes nothing of that tile).
template <typename IO, bool OUT, bool GATE, bool WRITE_GR = true>
__device__ __forceinline__ Rev exact_wave(const Chan& ch, const Carry& fin, const Rev& rin, const WaveRows& w,
                                          Rsrc gyr, Rsrc gkr, Rsrc gvr, Rsrc grr, int nv, bool valid, float& gw,
                                          float& gu) {
    Rev c = rin;
    const double w2 = w2_of(ch), u2 = u2_of(ch);
#pragma unroll 1
    for (int j = nv - 1; j >= 0; --j) {
        // forward state entering token j
        Carry st = fin;
#pragma unroll 1
        for (int i = 0; i < j; ++i) {
            const uint32_t so = (uint32_t)i * w.row_bytes;
            const float ki = valid ? load_elt<IO>(w.k, w.lane_off, so) : 0.f;
            const float vi = valid ? load_elt<IO>(w.v, w.lane_off, so) : 0.f;
            (void)lse_token<false>(ch, st, ki, vi);
        }
        const uint32_t so = (uint32_t)j * w.row_bytes;
        const float kj = valid ? load_elt<IO>(w.k, w.lane_off, so) : 0.f;
        const float vj = valid ? load_elt<IO>(w.v, w.lane_off, so) : 0.f;
        float gj = valid ? load_elt<IO>(gyr, w.lane_off, so) : 0.f;
        float rj = 0.f;
        if constexpr (GATE) {  // gj is dL/dz: dL/dy = dL/dz sigmoid(r)
            rj = valid ? load_elt<IO>(w.r, w.lane_off, so) : 0.f;
            gj *= sigmoid_f(rj);
        }
        // y_j and q_j = gy_j / D_j = qm 2^qe
        const double k2 = (double)kj * kLog2eD;
        const double uk = u2 + k2;
        const double qref = fmax(st.p, uk);
        const float e1 = ex2((float)(st.p - qref));
        const float e2 = ex2((float)(uk - qref));
        const float inv = rcp(fmaf(e1, st.b, e2));
        const float yj = fmaf(e1, st.a, e2 * vj) * inv;
        const float qm = gj * inv;
        if constexpr (GATE && !OUT && WRITE_GR)  // dL/dr, once (in the aggregate pass)
            if (valid) store_elt<IO>(grr, w.lane_off, so, gj * yj * sigmoid_f(-rj));
        const double qe = -qref;
        if (OUT) {
            const float ek = ex2((float)(k2 + c.r));         // e^{k_j} 2^r
            const float cur = ex2((float)(uk + qe)) * qm;   // e^{u+k_j} q_j
            const float dvy = vj - yj;
            const float dv = fmaf(ek, c.g, cur);
            const float dk = fmaf(ek, fmaf(vj, c.g, -c.h), cur * dvy);
            gw = fmaf(-ek, fmaf(vj, c.gp, -c.hp), gw);
            gu = fmaf(cur, dvy, gu);
            if (valid) {
                store_elt<IO>(gkr, w.lane_off, so, dk);
                store_elt<IO>(gvr, w.lane_off, so, dv);
            }
        }
        // reverse sums at the position before token j
        const double rd = c.r - w2;
        const double rn = fmax(rd, qe);
        const float f1 = ex2((float)(rd - rn));
        const float f2 = ex2((float)(qe - rn));
        c = normalize_rev(Rev{fmaf(f2, qm, f1 * c.g), fmaf(f2, qm * yj, f1 * c.h), f1 * (c.gp + c.g),
                              f1 * (c.hp + c.h), rn});
    }
    return c;
}

// Everything a tile's waves share.
template <int NW>
struct BwdShared {
    int ticket;
    float a[NW][64];  // forward: per-wave aggregate
    float b[NW][64];
    double p[NW][64];
    float g[NW][64];  // reverse: per-wave aggregate, then the carry after each wave
    float h[NW][64];
    float gp[NW][64];
    float hp[NW][64];
    double r[NW][64];
    float gw[NW][64];  // per-wave partial sums
    float gu[NW][64];
    float stash[4 * (kBwdTile / NW)][64];  // wave 0's chunk while it runs the look-back
};

// Fast-path bound for the reverse carry in a wave's frame: G^ = g 2^(r + R) with |g| < 1.
constexpr float kSpanRev = 60.f;

// Records of the backward scan: rec[chunk][g][slot][comp][lane] (u64; slot 0 the tile's
// reverse aggregate, slot 1 the inclusive carry at the tile's start; comp = g, h, gp, hp,
// r), status[g][chunk] as in the forward scan.
struct RevRecs {
    uint64_t* rec;       // records of chunk 0 of this group
    uint32_t* status;    // this group's status words
    size_t chunk_words;  // words per chunk index over all groups: n_groups * 10 * 64
    uint32_t tag_agg, tag_incl;
    uint32_t give_up_word;
    __device__ __forceinline__ uint64_t* word(int chunk, int slot, int comp, int lane) const {
        return rec + (size_t)chunk * chunk_words + (size_t)(slot * 5 + comp) * 64 + lane;
    }
};

__device__ __forceinline__ void publish_rev(const RevRecs& R, int chunk, int slot, int lane, const Rev& c,
                                            uint32_t tag) {
    st_word(R.word(chunk, slot, 0, lane), c.g, tag);
    st_word(R.word(chunk, slot, 1, lane), c.h, tag);
    st_word(R.word(chunk, slot, 2, lane), c.gp, tag);
    st_word(R.word(chunk, slot, 3, lane), c.hp, tag);
    st_word(R.word(chunk, slot, 4, lane), (float)c.r, tag);
    if (lane == 0) __hip_atomic_store(&R.status[chunk], tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The carry entering chunk ci from the right (ci < n_chunks - 1): folded from the
// nearest inclusive record on the right through the aggregates between, in chunk order
// from right to left, with advance_rev (every chunk between is a full tile).  The
// aggregates are read FB per round, their loads in flight together (one round trip for
// up to FB tiles of a chain that has fallen behind); each round re-reads its words until
// every tag matches; gives up like the forward scan.
template <int TILE, int FB>
__device__ __forceinline__ bool rev_look_back(const BwdArgs& args, const RevRecs& R, double w2, int ci, int lane,
                                              Rev& out) {
    // every poll reads the inclusive record of chunk ci+1, which ends the search at once when
    // complete, together with the status words of chunks ci+1 ... ci+64
    int start;
    for (uint32_t spin = 0;; ++spin) {
        uint64_t inc[5];
        bool good = true;
#pragma unroll
        for (int q = 0; q < 5; ++q) {
            inc[q] = ld_word(R.word(ci + 1, 1, q, lane));
            good = good && word_tag(inc[q]) == R.tag_incl;
        }
        const int pc = ci + 1 + lane;
        const uint32_t st = pc < args.n_chunks ? ld_status(&R.status[pc]) : 0u;
        if (__all(good)) {
            out = Rev{word_val(inc[0]), word_val(inc[1]), word_val(inc[2]), word_val(inc[3]), (double)word_val(inc[4])};
            return true;
        }
        start = scan_window<1>(st, pc < args.n_chunks, ci + 1, args.n_chunks - (ci + 1), R.tag_agg, R.tag_incl);
        if (start >= 0) break;
        if (start == kWindowAllReady) {  // 64 aggregates: continue the search beyond the window
            start = find_inclusive<1>(R.status, args.n_chunks, ci + 64, lane, R.tag_agg, R.tag_incl, args.ctrl,
                                      R.give_up_word);
            if (start < 0) return false;
            break;
        }
        if (must_stop(args.ctrl, R.give_up_word, spin)) return raise_give_up(args.ctrl, R.give_up_word, lane);
        __builtin_amdgcn_s_sleep(kPollSleep);
    }
    // fold from the inclusive record of `start` through the aggregates before it, FB per round
    // (chunks c0, c0 - 1, ...); the first round also loads the inclusive record, and a round
    // re-reads its words until every tag matches
    Rev P{0.f, 0.f, 0.f, 0.f, 0.0};
    bool have_p = false;
#pragma unroll 1
    for (int c0 = start - 1;;) {
        const int n = min(FB, c0 - ci);
        uint64_t inc[5], t[FB][5];
        for (uint32_t spin = 0;; ++spin) {
            bool good = true;
            if (!have_p)
#pragma unroll
                for (int q = 0; q < 5; ++q) {
                    inc[q] = ld_word(R.word(start, 1, q, lane));
                    good = good && word_tag(inc[q]) == R.tag_incl;
                }
#pragma unroll
            for (int j = 0; j < FB; ++j)
                if (j < n)
#pragma unroll
                    for (int q = 0; q < 5; ++q) {
                        t[j][q] = ld_word(R.word(c0 - j, 0, q, lane));
                        good = good && word_tag(t[j][q]) == R.tag_agg;
                    }
            if (__all(good)) break;
            if (must_stop(args.ctrl, R.give_up_word, spin)) return raise_give_up(args.ctrl, R.give_up_word, lane);
            __builtin_amdgcn_s_sleep(kPollSleep);
        }
        if (!have_p) {
            P = Rev{word_val(inc[0]), word_val(inc[1]), word_val(inc[2]), word_val(inc[3]), (double)word_val(inc[4])};
            have_p = true;
        }
#pragma unroll
        for (int j = 0; j < FB; ++j)
            if (j < n)
                P = advance_rev(P, Rev{word_val(t[j][0]), word_val(t[j][1]), word_val(t[j][2]), word_val(t[j][3]),
                                       (double)word_val(t[j][4])},
                                TILE, w2);
        c0 -= n;
        if (c0 <= ci) break;
    }
    out = P;
    return true;
}

// The reverse carry entering chunk ci from the right (ci < n_chunks - 1) without waiting on
// any other tile, for a tile whose look-back gave up or a launch forced onto that path: from
// the nearest chunk to the right whose inclusive record is complete (else the end of the
// sequence, where no later output contributes), leftwards through every chunk between, by
// its aggregate record when that is complete, else by walking the chunk's tokens backwards
// from memory with the exact per-token path, its forward state taken from the state dumped
// at the chunk's start.  Every record word used is validated by its own tag; nothing is
// waited for.  seq_off: byte offset of this group at time step 0; li: this lane's index.
template <typename IO, int TILE, bool GATE>
__device__ __forceinline__ Rev rebuild_rev(const BwdArgs& args, const RevRecs& R, const Chan& ch, int ci, int lane,
                                           size_t seq_off, uint32_t lane_off, bool cvalid, size_t li) {
    const double w2 = w2_of(ch);
    int start = args.n_chunks;
    Rev P = rev_rec_form(empty_rev());
    for (int nearest = ci + 1; nearest < args.n_chunks && start == args.n_chunks; nearest += 64) {
        const int pc = nearest + lane;
        const uint32_t st = pc < args.n_chunks ? ld_status(&R.status[pc]) : 0u;
        uint64_t cand = __ballot(pc < args.n_chunks && st == R.tag_incl);
        while (cand) {
            const int d = __builtin_ctzll(cand);
            uint64_t wds[5];
            bool good = true;
#pragma unroll
            for (int q = 0; q < 5; ++q) {
                wds[q] = ld_word(R.word(nearest + d, 1, q, lane));
                good = good && word_tag(wds[q]) == R.tag_incl;
            }
            if (__all(good)) {
                start = nearest + d;
                P = Rev{word_val(wds[0]), word_val(wds[1]), word_val(wds[2]), word_val(wds[3]), (double)word_val(wds[4])};
                break;
            }
            cand &= cand - 1ull;
        }
    }
    const uint32_t row_bytes = (uint32_t)((size_t)args.C * sizeof(IO));
    constexpr int kHalf = TILE / 2;
    static_assert(kHalf <= 64, "exact walks address at most 64 rows from one resource");
#pragma unroll 1
    for (int m = start - 1; m > ci; --m) {
        const int len = min(TILE, args.T - m * TILE);
        uint64_t t[5];
        bool good = true;
#pragma unroll
        for (int q = 0; q < 5; ++q) {
            t[q] = ld_word(R.word(m, 0, q, lane));
            good = good && word_tag(t[q]) == R.tag_agg;
        }
        if (__all(good)) {
            P = advance_rev(P, Rev{word_val(t[0]), word_val(t[1]), word_val(t[2]), word_val(t[3]), (double)word_val(t[4])},
                            len, w2);
            continue;
        }
        const size_t ti = (size_t)m * args.n_lanes + li;
        const Carry fin = normalize(Carry{args.fw_a[ti], args.fw_b[ti], (double)args.fw_p[ti]});
        Rev c = normalize_rev(P);
        float gw = 0.f, gu = 0.f;  // not used by the aggregate pass
        for (int half = len > kHalf ? 1 : 0; half >= 0; --half) {
            const size_t off = seq_off + ((size_t)m * TILE + (size_t)half * kHalf) * row_bytes;
            Carry fh = fin;
            if (half)
                walk_rows_exact<IO>(ch, fh, static_cast<const char*>(args.k) + seq_off + (size_t)m * TILE * row_bytes,
                                    static_cast<const char*>(args.v) + seq_off + (size_t)m * TILE * row_bytes, lane_off,
                                    row_bytes, kHalf, cvalid);
            WaveRows rows;
            rows.k = make_rsrc(static_cast<const char*>(args.k) + off);
            rows.v = make_rsrc(static_cast<const char*>(args.v) + off);
            rows.y = rows.k;
            rows.r = GATE ? make_rsrc(static_cast<const char*>(args.r) + off) : rows.k;
            rows.lane_off = lane_off;
            rows.row_bytes = row_bytes;
            rows.pair_off = 0;
            rows.upper = 0;
            rows.partner = 0;
            const Rsrc gyr = make_rsrc(static_cast<const char*>(args.gy) + off);
            const int nvh = half ? len - kHalf : min(len, kHalf);
            c = exact_wave<IO, false, GATE, false>(ch, fh, c, rows, gyr, gyr, gyr, gyr, nvh, cvalid, gw, gu);
        }
        P = rev_rec_form(normalize_rev(c));
    }
    return P;
}

// One tile of the backward scan (see the plan at the top).  Tiles are numbered in the
// order workgroups start, from the last chunk of the sequence to the first, so every
// tile this one waits on has started and publishes its aggregate without waiting.
// Aggregates folded per look-back round (wave 0's chunk is stashed in LDS by then, so the
// 40 registers of four records are free; 4 against 1: the same bits, 0.4-0.5% faster for
// bf16, B=1, T=65536, C=5120).
constexpr int kRevFoldBatch = 4;

template <typename IO, int L, int NW, bool GATE>
__global__ __launch_bounds__(64 * NW, 4) void bwd_scan_kernel(BwdArgs args) {
    constexpr int TILE = L * NW;
    static_assert(TILE == kBwdTile, "tiles must line up with the dumped forward tiles");
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int C = args.C, T = args.T;
    __shared__ BwdShared<NW> sh;

    if (threadIdx.x == 0) sh.ticket = (int)atomicAdd(&args.ctrl[kCtrlTicket], 1u);
    __syncthreads();
    bool forced = false;
    const int ticket = (int)remap_ticket((uint32_t)__builtin_amdgcn_readfirstlane(sh.ticket),
                                         (uint32_t)args.n_groups * (uint32_t)args.n_chunks, args.ctrl, forced);
    const int g = ticket % args.n_groups;
    const int ci = args.n_chunks - 1 - ticket / args.n_groups;
    const int bi = g / args.groups_per_row;
    const int c_grp = (g - bi * args.groups_per_row) * 64;
    const int c = c_grp + (kPair<IO> ? pair_channel(lane) : lane);
    const bool cvalid = c < C;
    const int t_tile = ci * TILE;
    const int tile_len = min(TILE, T - t_tile);
    const int t0 = __builtin_amdgcn_readfirstlane(t_tile + wid * L);
    const int nv = max(0, min(L, T - t0));
    const size_t li = (size_t)g * 64 + (c - c_grp);    // lane index (this lane's channel)
    const size_t ti = (size_t)ci * args.n_lanes + li;  // (tile, lane) index
    const size_t plane = (size_t)args.plane;

    WaveRows rows;
    const size_t off = (((size_t)bi * T + (size_t)min(t0, T)) * C + c_grp) * sizeof(IO);
    rows.k = make_rsrc(static_cast<const char*>(args.k) + off);
    rows.v = make_rsrc(static_cast<const char*>(args.v) + off);
    rows.y = make_rsrc(static_cast<char*>(args.gk) + off);  // unused by the row helpers here
    rows.lane_off = (uint32_t)((c - c_grp) * sizeof(IO));
    rows.row_bytes = (uint32_t)(C * sizeof(IO));
    rows.pair_off = (uint32_t)((lane & 31) * 4) + (uint32_t)(lane >> 5) * rows.row_bytes;
    rows.upper = (uint32_t)(lane >> 5);
    rows.partner = (uint32_t)((lane ^ 32) << 2);
    const Rsrc gyr = make_rsrc(static_cast<const char*>(args.gy) + off);
    const Rsrc gkr = make_rsrc(static_cast<char*>(args.gk) + off);
    const Rsrc gvr = make_rsrc(static_cast<char*>(args.gv) + off);
    Rsrc grr = gkr;
    if constexpr (GATE) {
        rows.r = make_rsrc(static_cast<const char*>(args.r) + off);
        grr = make_rsrc(static_cast<char*>(args.gr) + off);
    }

    BwdChunk<L> ck;
    ck.template load<IO>(rows, gyr, nv, cvalid);
    // the forward state entering the tile (every wave starts its prefix from it)
    const float fwa = args.fw_a[ti], fwb = args.fw_b[ti], fwp = args.fw_p[ti];
    float sr[GATE ? L : 1];  // gate: r rows, then dL/dr
    if constexpr (GATE) BwdChunk<L>::template load_rows<IO>(rows, rows.r, cvalid && nv == L, sr);

    // read after the loads are issued; constant during the launch
    const uint32_t epoch = __builtin_amdgcn_readfirstlane(args.ctrl[kCtrlEpoch]);
    RevRecs recs;
    recs.rec = static_cast<uint64_t*>(args.rrecs) + (size_t)g * 10 * 64;
    recs.chunk_words = (size_t)args.n_groups * 10 * 64;
    recs.status = args.status + (size_t)g * args.n_chunks;
    recs.tag_agg = (epoch << 2) | kKindAgg;
    recs.tag_incl = (epoch << 2) | kKindIncl;
    recs.give_up_word = epoch | kCtrlGiveUpMark;
    forced = forced || launch_forced(args.ctrl);

    const Chan ch = make_chan(args.w[cvalid ? c : 0], args.u[cvalid ? c : 0]);
    const double w2 = w2_of(ch);
    float kmax, kmin;
    ck.range(kmax, kmin);
    const float R = kmax * kLog2e;
    const bool fast = __all(nv == L && chunk_fast_ok(ch, kmax, kmin));

    // ---- forward: per-wave aggregate, combined into the state before each wave ----
    Carry agg = empty_carry();
    if (fast) {
        agg = ck.aggregate(ch, R);
    } else {
        lse_walk<IO, false>(ch, agg, rows, nv, cvalid, false);
    }
    sh.a[wid][lane] = agg.a;
    sh.b[wid][lane] = agg.b;
    sh.p[wid][lane] = agg.p;
    __syncthreads();
    // wave 0 reads the next tile's inclusive record now; by the look-back it has usually arrived
    // complete, and the look-back is then skipped
    const bool has_next = ci + 1 < args.n_chunks;
    uint64_t nx[5];
#pragma unroll
    for (int q = 0; q < 5; ++q) nx[q] = (wid == 0 && has_next) ? ld_word(recs.word(ci + 1, 1, q, lane)) : 0ull;
    // the forward state entering this wave: the tile's state followed by the waves before it,
    // in wave order (every wave folds its own prefix; none waits for another)
    Carry fin = normalize(Carry{fwa, fwb, (double)fwp});
#pragma unroll 1
    for (int wv = 0; wv < wid; ++wv) {
        const int nvw = max(0, min(L, T - (t_tile + wv * L)));
        const Carry aw{sh.a[wv][lane], sh.b[wv][lane], sh.p[wv][lane]};
        fin = normalize(combine(fin, aw, (double)nvw * w2));
    }

    // ---- per-wave reverse aggregate (from nothing after the wave) ----
    const bool wave_fast = fast && __all(fin.p - (double)R <= (double)kSpan);
    float gw = 0.f, gu = 0.f;
    Rev ragg;
    if (wave_fast) {
        if constexpr (GATE) {
            ck.forward_gated(ch, fin, R, sr);
            BwdChunk<L>::template store_rows<IO>(rows, grr, cvalid, sr);
        } else {
            ck.forward(ch, fin, R);
        }
        ragg = ck.reverse_aggregate(ch, R);
    } else {
        ragg = exact_wave<IO, false, GATE>(ch, fin, empty_rev(), rows, gyr, gkr, gvr, grr, nv, cvalid, gw, gu);
    }
    ragg = normalize_rev(ragg);
    sh.g[wid][lane] = ragg.g;
    sh.h[wid][lane] = ragg.h;
    sh.gp[wid][lane] = ragg.gp;
    sh.hp[wid][lane] = ragg.hp;
    sh.r[wid][lane] = ragg.r;
    __syncthreads();

    // ---- wave 0: the suffix aggregates (slot wv: waves wv .. NW-1), the tile aggregate (the
    // suffix from wave 0), look-back, publish; the carry entering from the right goes to LDS ----
    if (wid == 0) {
        ck.stash(sh.stash, lane);
        asm volatile("" ::: "memory");  // the chunk must really leave the registers
        Rev rw[NW];  // every wave's aggregate read at once (the stashed chunk's registers are free)
#pragma unroll
        for (int wv = 0; wv < NW; ++wv)
            rw[wv] = Rev{sh.g[wv][lane], sh.h[wv][lane], sh.gp[wv][lane], sh.hp[wv][lane], sh.r[wv][lane]};
        Rev run = empty_rev();
#pragma unroll
        for (int wv = NW - 1; wv >= 0; --wv) {
            const int nvw = max(0, min(L, T - (t_tile + wv * L)));
            run = normalize_rev(fold_rev(rw[wv], run, nvw, w2));
            if (wv > 0) {
                sh.g[wv][lane] = run.g;
                sh.h[wv][lane] = run.h;
                sh.gp[wv][lane] = run.gp;
                sh.hp[wv][lane] = run.hp;
                sh.r[wv][lane] = run.r;
            }
        }
        const Rev agg_rec = rev_rec_form(run);
        Rev rin = rev_rec_form(empty_rev());
        if (has_next) {
            bool ready = !forced;
#pragma unroll
            for (int q = 0; q < 5; ++q) ready = ready && word_tag(nx[q]) == recs.tag_incl;
            bool have = false;
            if (__all(ready)) {
                rin = Rev{word_val(nx[0]), word_val(nx[1]), word_val(nx[2]), word_val(nx[3]), (double)word_val(nx[4])};
                have = true;
            } else if (!forced) {
                publish_rev(recs, ci, 0, lane, agg_rec, recs.tag_agg);
                have = rev_look_back<TILE, kRevFoldBatch>(args, recs, w2, ci, lane, rin);
            } else {
                raise_give_up(args.ctrl, recs.give_up_word, lane);
            }
            if (!have)
                rin = rebuild_rev<IO, TILE, GATE>(args, recs, ch, ci, lane, ((size_t)bi * T * C + c_grp) * sizeof(IO),
                                                  rows.lane_off, cvalid, li);
        }
        if (ci > 0) publish_rev(recs, ci, 1, lane, advance_rev(rin, agg_rec, tile_len, w2), recs.tag_incl);
        rin = normalize_rev(rin);
        sh.g[0][lane] = rin.g;  // slot 0 (the tile aggregate is not needed again) takes the carry
        sh.h[0][lane] = rin.h;
        sh.gp[0][lane] = rin.gp;
        sh.hp[0][lane] = rin.hp;
        sh.r[0][lane] = rin.r;
        asm volatile("" ::: "memory");
        ck.unstash(sh.stash, lane);
    }
    __syncthreads();

    // ---- gradients of this wave's tokens from the carry after the wave: the carry entering
    // the tile from the right folded through the waves after this one (their suffix aggregate)
    Rev cin{sh.g[0][lane], sh.h[0][lane], sh.gp[0][lane], sh.hp[0][lane], sh.r[0][lane]};
    if (wid + 1 < NW) {
        const int n_after = max(0, min(TILE - (wid + 1) * L, T - (t_tile + (wid + 1) * L)));
        const Rev suf{sh.g[wid + 1][lane], sh.h[wid + 1][lane], sh.gp[wid + 1][lane], sh.hp[wid + 1][lane],
                      sh.r[wid + 1][lane]};
        cin = normalize_rev(fold_rev(suf, cin, n_after, w2));
    }
    if (wave_fast && __all(cin.r + (double)R <= (double)kSpanRev)) {
        ck.backward(ch, cin, R, gw, gu);
        ck.template store_grads<IO>(rows, gkr, gvr, cvalid);
    } else {
        gw = 0.f;
        gu = 0.f;
        (void)exact_wave<IO, true, GATE>(ch, fin, cin, rows, gyr, gkr, gvr, grr, nv, cvalid, gw, gu);
    }
    sh.gw[wid][lane] = gw;
    sh.gu[wid][lane] = gu;
    __syncthreads();
    if (wid == 0) {
        float sw = 0.f, su = 0.f;
#pragma unroll
        for (int wv = 0; wv < NW; ++wv) {
            sw += sh.gw[wv][lane];
            su += sh.gu[wv][lane];
        }
        args.part[ti] = sw;
        args.part[plane + ti] = su;
    }
    // ---- launch bookkeeping (a give-up of the forward scan before is carried over) ----
    if (threadIdx.x == 0)
        finish_tile(args.ctrl, (uint32_t)args.n_groups * (uint32_t)args.n_chunks, epoch, args.inherit_give_up);
}

// dL/dw and dL/du per lane: the tiles' partials summed in a fixed order.  Block: 64 lanes
// x kRedSlices slices; slice s sums chunks s, s + kRedSlices, ...; slice 0 then adds the
// slices' sums in order.
constexpr int kRedSlices = 16;

__global__ __launch_bounds__(64 * kRedSlices) void bwd_reduce_kernel(BwdArgs args) {
    __shared__ float sw_s[kRedSlices][64], su_s[kRedSlices][64];
    const int lane = threadIdx.x & 63, slice = threadIdx.x >> 6;
    const long li = (long)blockIdx.x * 64 + lane;
    const size_t plane = (size_t)args.plane;
    float sw = 0.f, su = 0.f;
    for (int ci = slice; ci < args.n_chunks; ci += kRedSlices) {
        sw += args.part[(size_t)ci * args.n_lanes + li];
        su += args.part[plane + (size_t)ci * args.n_lanes + li];
    }
    sw_s[slice][lane] = sw;
    su_s[slice][lane] = su;
    __syncthreads();
    if (slice != 0) return;
    const int g = (int)(li / 64);
    const int bi = g / args.groups_per_row;
    const int c = (g % args.groups_per_row) * 64 + lane;
    if (c >= args.C) return;
    sw = 0.f;
    su = 0.f;
#pragma unroll
    for (int s = 0; s < kRedSlices; ++s) {
        sw += sw_s[s][lane];
        su += su_s[s][lane];
    }
    args.gw[(size_t)bi * args.C + c] = sw;
    args.gu[(size_t)bi * args.C + c] = su;
}

template <typename IO>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t s) {
    constexpr int L = 16, NW = kBwdTile / L;
    const unsigned tiles = (unsigned)((long)a.n_groups * a.n_chunks);
    if (a.r)
        hipLaunchKernelGGL((bwd_scan_kernel<IO, L, NW, true>), dim3(tiles), dim3(64 * NW), 0, s, a);
    else
        hipLaunchKernelGGL((bwd_scan_kernel<IO, L, NW, false>), dim3(tiles), dim3(64 * NW), 0, s, a);
    hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)a.n_groups), dim3(64 * kRedSlices), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a, int io, hipStream_t s) {
    if (io == kIoF32) return launch_bwd_t<float>(a, s);
    if (io == kIoBf16Pair) return launch_bwd_t<Bf16Pair>(a, s);
    return launch_bwd_t<uint16_t>(a, s);
}

}  // namespace wkv
