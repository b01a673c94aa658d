/*
 * libwkv -- the RWKV-4 time-mixing WKV operator for AMD MI355X (gfx950).
 *
 * The operation (page "Reinventing RNNs for the Transformer Era: RWKV", a paper
 * review on velog; section "WKV 연산자", WKV equation), for every batch b,
 * channel c and time t = 1..T:
 *
 *   y_t = ( sum_{i<t} e^{-(t-1-i) w + k_i} v_i + e^{u + k_t} v_t )
 *         / ( sum_{i<t} e^{-(t-1-i) w + k_i} + e^{u + k_t} )
 *
 * with w (the decay rate itself, applied as e^{-w}) and u (the bonus of the
 * current token) per channel.  Section "RNN-유사추론" of the same page gives
 * the RNN form y_t = (A_t + e^{u+k_t} v_t) / (B_t + e^{u+k_t}) with a
 * per-channel state (A_t, B_t) carried to the next token (its decoding list,
 * steps 4 and 7).  This library advances the state as
 * A_{t+1} = e^{-w} A_t + e^{k_t} v_t, B_{t+1} = e^{-w} B_t + e^{k_t}, the
 * reading that reproduces the WKV equation.
 *
 * State triples.  A state is stored as three float32 arrays (a, b, p) meaning
 * A = a * e^p and B = b * e^p.  The representation is not unique: (a e^d,
 * b e^d, p - d) is the same state, so compare log B = p + log b and A / B.
 * The empty state (no past) is a = b = 0, p = WKV_P_EMPTY.
 *
 * Conventions for every entry point
 *  - Pointers are DEVICE pointers on the current HIP device; the caller owns
 *    every buffer.  Tensors are dense and row-major with the channel index
 *    fastest: k, v, y are [B, T, C] (forward) or [N, G, C] (step).
 *  - Calls are asynchronous on `stream` (0 = the null stream) and never
 *    allocate; only wkv_forward_workspace_query synchronises.  The library
 *    keeps no state of its own: what a chunked forward call carries to the
 *    next one (a launch counter) lives in the caller's workspace.
 *  - Every call except wkv_forward_workspace_query may be captured in a HIP
 *    graph: workspace counters are set by kernels (no hipMemsetAsync), and
 *    each chained-scan launch leaves them ready for the next, so a replay
 *    behaves as the same launch made eagerly.
 *  - Pointers cannot be checked for being device memory: passing host
 *    memory faults the GPU.  The Python binding refuses such tensors.
 *  - All argument checks happen before any HIP call.  A negative size, or a
 *    NULL pointer for a non-empty operand, gives WKV_EINVAL; an unknown dtype
 *    gives WKV_EDTYPE; a workspace smaller than the query gives
 *    WKV_EWORKSPACE; a failed launch gives WKV_EHIP.  Any zero size returns
 *    WKV_OK without touching the GPU.
 *  - y must not alias k or v (not detected).  NaN and Inf in the inputs
 *    propagate to the outputs; nothing traps.
 *  - The scan kernels address up to 64 rows of C elements from one 32-bit
 *    window: C * (bytes per element) * 64 must not exceed 2^31 - 1 (C below
 *    2^23 for float32, 2^24 for bfloat16); wider rows give WKV_EINVAL.
 *  - Results are bitwise reproducible for a given shape, dtype, algorithm
 *    and chunk length.
 */
#ifndef LIBWKV_H
#define LIBWKV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum wkv_status {
    WKV_OK = 0,
    WKV_EINVAL = 1,     /* bad size, NULL pointer, bad algorithm or chunk length */
    WKV_EDTYPE = 2,     /* unknown dtype */
    WKV_EWORKSPACE = 3, /* workspace missing or too small */
    WKV_EHIP = 4        /* a HIP launch failed */
} wkv_status;

/* dtype of k, v and y.  w, u and the state (a, b, p) are always float32, and
 * all arithmetic is float32 with float64 exponent bookkeeping. */
typedef enum wkv_dtype {
    WKV_F32 = 0,
    WKV_BF16 = 1 /* bfloat16; y is rounded to nearest-even */
} wkv_dtype;

/* How wkv_forward_ex computes the time recurrence. */
typedef enum wkv_algo {
    WKV_ALGO_AUTO = 0,    /* chunked, except SEQ for T <= 64 (and B <= 65535) */
    WKV_ALGO_SEQ = 1,     /* one thread walks all of T for its channels */
    WKV_ALGO_CHUNKED = 2  /* T split into chunks, single-pass chained scan */
} wkv_algo;

/* p of the empty state (a = b = 0). */
#define WKV_P_EMPTY (-1.0e38f)

/* Chunk lengths (time steps per workgroup tile) accepted by the chunked
 * algorithm; 0 selects 256 (512 for problems of fewer than 1024 tiles of 256, and
 * for bfloat16 moved as row pairs: even C, 4-byte aligned arrays). */
#define WKV_CHUNK_LENS {64, 128, 256, 512}

/*
 * Bytes of device workspace that wkv_forward_ex needs for this problem with
 * this algorithm and chunk length (0 for the sequential algorithm).  The same
 * value serves wkv_forward (algo AUTO, chunk_len 0) and wkv_forward_state.
 * Returns 0 for empty problems and (size_t)-1 for invalid arguments.
 */
size_t wkv_forward_workspace_bytes(int64_t B, int64_t T, int64_t C, wkv_dtype dt,
                                   wkv_algo algo, int64_t chunk_len);

/*
 * Zero-fill a forward workspace (asynchronously, on `stream`).  Every
 * workspace must start zero-filled -- through this call or any other fill
 * with zeros -- before its first use by wkv_forward*; the forward calls keep
 * it valid afterwards, for any later problem size that fits.  ws_bytes must
 * be a multiple of 4 and ws 4-byte aligned (WKV_EINVAL otherwise).
 */
wkv_status wkv_forward_workspace_init(void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Diagnostics of a forward workspace, read after the calls queued on `stream`
 * have finished (this call synchronises `stream`):
 *   *gave_up : non-zero if the last chunked call on this workspace had a tile
 *              stop waiting for another (its bounded spin ran out, another tile
 *              of the call had stopped, the call was forced onto that path by
 *              wkv_workspace_force_give_up, or the workspace's ticket counter
 *              was not zero when the call started).  Such a tile rebuilds the
 *              state it needs without waiting (from the complete records and
 *              the inputs in memory), so the outputs stay valid; the flag only
 *              says that the slower path ran.
 *   *epoch   : launch counter of the chunked calls made on this workspace.
 * WKV_EINVAL for NULL pointers, WKV_EWORKSPACE if ws_bytes cannot hold the
 * control block, WKV_EHIP if the synchronisation or copy fails.
 */
wkv_status wkv_forward_workspace_query(const void* ws, size_t ws_bytes, uint32_t* gave_up,
                                       uint32_t* epoch, hipStream_t stream);

/*
 * Test hook of the give-up path of the chained scans (wkv_forward*,
 * wkv_backward*, wkv_linear_attention* in one pass): the next `launches`
 * chained-scan launches on this workspace (a recomputing wkv_backward makes
 * two) run every tile as if each of its waits had given up at once, so every
 * tile rebuilds its entering state from the complete records and the inputs
 * in memory.  Results stay within the stated tolerances (they are no longer
 * bitwise those of the usual path), and the calls are slower.  Asynchronous
 * on `stream`, no allocation.  ws as for wkv_forward_workspace_query
 * (WKV_EINVAL for NULL, WKV_EWORKSPACE if it cannot hold the control block).
 */
wkv_status wkv_workspace_force_give_up(void* ws, size_t ws_bytes, uint32_t launches, hipStream_t stream);

/*
 * Whole-sequence WKV (the page's time-parallel training mode, section
 * "Transformer-유사학습": every op runs over batch and time at once and only
 * WKV runs as a scan).
 *   w, u : [C] float32 device arrays.
 *   k, v : [B, T, C] device arrays of dtype dt (read only).
 *   y    : [B, T, C] device array of dtype dt (written).
 *   ws   : device workspace of at least wkv_forward_workspace_bytes(...)
 *          bytes, zero-filled before its first use (wkv_forward_workspace_init)
 *          and then owned by the library between calls: the chunked scan keeps
 *          a launch counter and per-tile records there.  One workspace must not
 *          be used by two calls that may run at the same time.
 * Starts every lane from the empty state.
 */
wkv_status wkv_forward(int64_t B, int64_t T, int64_t C, wkv_dtype dt,
                       const float* w, const float* u,
                       const void* k, const void* v, void* y,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * wkv_forward for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): no workspace
 * argument and no allocation of any kind.  The chunked scan's workspace is a
 * static device array of 32 MiB that the library holds on every GPU it runs
 * on until the process ends; the first call on a device looks up its address
 * (hipGetSymbolAddress, with that device current) and clears its launch
 * counters with a small kernel on `stream`.  Same kernels and results as
 * wkv_forward.  A problem whose workspace (wkv_forward_workspace_bytes with
 * WKV_ALGO_AUTO, chunk 0) exceeds 32 MiB runs the sequential algorithm (as
 * wkv_forward_ex with WKV_ALGO_SEQ, which needs no workspace), or, with
 * B > 65535 (beyond its grid), gives WKV_EWORKSPACE before any launch.  All calls on one GPU share that GPU's array, which keeps the last
 * call's records: calls that may overlap in time on the same GPU (other
 * streams, other host threads) race and must not be made.  Other arguments
 * and errors as wkv_forward.
 */
wkv_status wkv_forward_noalloc(int64_t B, int64_t T, int64_t C, wkv_dtype dt,
                               const float* w, const float* u,
                               const void* k, const void* v, void* y, hipStream_t stream);

/* wkv_forward with an explicit algorithm and chunk length (0 = default). */
wkv_status wkv_forward_ex(int64_t B, int64_t T, int64_t C, wkv_dtype dt,
                          const float* w, const float* u,
                          const void* k, const void* v, void* y,
                          void* ws, size_t ws_bytes,
                          wkv_algo algo, int64_t chunk_len, hipStream_t stream);

/*
 * Whole-sequence WKV that starts from a given state and returns the final
 * one: the prefill that hands over to wkv_step (the page's time-parallel mode
 * joined to its time-sequential mode; the state after token T is the one the
 * decoding loop stores for token T+1).
 *   state_in_a/b/p  : [B, C] float32 device arrays, or all three NULL for the
 *                     empty state.
 *   state_out_a/b/p : [B, C] float32 device arrays written with the state
 *                     after the last token, or all three NULL.  They may be
 *                     the same arrays as state_in_*.
 * The other arguments are those of wkv_forward_ex.  With T = 0 the state is
 * copied through (a launch is made only when in and out differ).
 */
wkv_status wkv_forward_state(int64_t B, int64_t T, int64_t C, wkv_dtype dt,
                             const float* w, const float* u,
                             const void* k, const void* v, void* y,
                             const float* state_in_a, const float* state_in_b,
                             const float* state_in_p,
                             float* state_out_a, float* state_out_b, float* state_out_p,
                             void* ws, size_t ws_bytes,
                             wkv_algo algo, int64_t chunk_len, hipStream_t stream);

/*
 * Bytes of device workspace that wkv_backward needs for this problem (0 for
 * empty problems, (size_t)-1 for invalid arguments): about one byte per
 * element of k (the records of a forward scan and of a backward scan over
 * tiles of 128 time steps, and five float32 values per such tile and channel).
 */
size_t wkv_backward_workspace_bytes(int64_t B, int64_t T, int64_t C, wkv_dtype dt);

/*
 * Gradients of the whole-sequence WKV for the page's time-parallel training
 * mode (section "Transformer-유사학습" trains through the WKV equation of
 * section "WKV 연산자"): given gy = dL/dy for y = WKV(w, u, k, v) started from
 * the empty state, writes
 *   gk, gv : [B, T, C] device arrays of dtype dt, dL/dk and dL/dv;
 *   gw, gu : [B, C] float32 device arrays, dL/dw and dL/du per lane (the
 *            gradient of the shared [C] parameter is the sum over b).
 * w, u, k, v are the forward inputs (the forward is recomputed; y is not
 * needed), gy is [B, T, C] of dtype dt.  The outputs must not alias the
 * inputs.  ws: device workspace of at least wkv_backward_workspace_bytes(...)
 * bytes, zero-filled before its first use (wkv_forward_workspace_init fills
 * any workspace) and owned by the library between calls; it starts with the
 * same control block as a forward workspace, so wkv_forward_workspace_query
 * reports on the last call (gave_up if either of its two scans, forward then
 * backward in time, gave up; each call advances the epoch by two).  One
 * workspace must not serve two calls that may run at the same time.  With
 * T = 0, gw and gu are zero-filled.  Deterministic: no atomics take part in
 * any sum.
 */
wkv_status wkv_backward(int64_t B, int64_t T, int64_t C, wkv_dtype dt,
                        const float* w, const float* u,
                        const void* k, const void* v, const void* gy,
                        void* gk, void* gv, float* gw, float* gu,
                        void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Training pair that skips the backward's forward scan.  wkv_forward_save is
 * wkv_forward_ex with the chunked algorithm at the default chunk length (its
 * workspace: wkv_forward_workspace_bytes(B, T, C, dt, WKV_ALGO_CHUNKED, 0))
 * that also writes, into `saved`, the state entering every 128th time step of
 * every lane: wkv_saved_states_bytes(B, T, C) bytes of device memory (about
 * 0.1 byte per element of k; opaque; (size_t)-1 for invalid sizes, 0 for
 * empty problems).  wkv_backward_saved then gives what wkv_backward gives for
 * the same w, u, k, v, gy, reading those states instead of recomputing them;
 * its workspace is wkv_backward_workspace_bytes(...).  The gradients are
 * bitwise those of wkv_backward.  A `saved` NULL or smaller than the query
 * gives WKV_EINVAL.
 */
size_t wkv_saved_states_bytes(int64_t B, int64_t T, int64_t C);

wkv_status wkv_forward_save(int64_t B, int64_t T, int64_t C, wkv_dtype dt,
                            const float* w, const float* u,
                            const void* k, const void* v, void* y,
                            float* saved, size_t saved_bytes,
                            void* ws, size_t ws_bytes, hipStream_t stream);

wkv_status wkv_backward_saved(int64_t B, int64_t T, int64_t C, wkv_dtype dt,
                              const float* w, const float* u,
                              const void* k, const void* v, const void* gy,
                              const float* saved, size_t saved_bytes,
                              void* gk, void* gv, float* gw, float* gu,
                              void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * The time-mixing block around WKV (page "Reinventing RNNs for the Transformer
 * Era: RWKV", sections "토큰 변환" and "출력 게이팅"); the dense projections
 * between them (W_r, W_k, W_v before, W_o after) are not part of this library.
 *
 * wkv_token_shift: the inputs of the R, K, V projections, a per-channel linear
 * interpolation between the current and the previous time step:
 *   out[m, b, t, c] = mu[m, c] x[b, t, c] + (1 - mu[m, c]) x[b, t-1, c],
 * for m < M (1 <= M <= 4, else WKV_EINVAL), x[b, -1, c] = x_prev[b, c] (the last
 * token of the previous call when a sequence continues) or 0 when x_prev is
 * NULL.  x: [B, T, C] dtype dt; x_prev: [B, C] dtype dt or NULL; mu: [M, C]
 * float32; out: [M, B, T, C] dtype dt, must not alias x.
 */
wkv_status wkv_token_shift(int64_t B, int64_t T, int64_t C, wkv_dtype dt,
                           const void* x, const void* x_prev, const float* mu,
                           int64_t M, void* out, hipStream_t stream);

/*
 * Backward of wkv_token_shift (page "Reinventing RNNs for the Transformer Era: RWKV", section
 * "토큰 변환", the interpolation the time-mixing block trains through): for
 * L = sum_m sum g_m * out_m,
 *   gx[b, t, c]   = sum_m mu_m[c] g_m[b, t, c] + (1 - mu_m[c]) g_m[b, t+1, c]   (g at t = T is 0)
 *   gmu[m, b, c]  = sum_t g_m[b, t, c] (x[b, t, c] - x[b, t-1, c])             (per lane, float32;
 *                   the [M, C] parameter's gradient is the sum over b)
 *   gprev[b, c]   = sum_m (1 - mu_m[c]) g_m[b, 0, c]                            (dL/dx_prev)
 * with x[b, -1, c] = x_prev[b, c] (zero when x_prev is NULL).  x [B, T, C], g [M, B, T, C],
 * gx [B, T, C] and gprev [B, C] are of dtype dt; mu [M, C] float32; 1 <= M <= 4; gprev may
 * be NULL (not wanted).  ws: device workspace of at least
 * wkv_token_shift_backward_workspace_bytes(B, T, C, M) bytes (no initialisation needed): the
 * per-segment partial sums of gmu, added per lane in a fixed order in float64, so results are
 * bitwise reproducible.  T = 0 writes zero gmu (and gprev).  Errors as wkv_token_shift, plus
 * WKV_EWORKSPACE.
 */
size_t wkv_token_shift_backward_workspace_bytes(int64_t B, int64_t T, int64_t C, int64_t M);
wkv_status wkv_token_shift_backward(int64_t B, int64_t T, int64_t C, wkv_dtype dt, const void* x,
                                    const void* x_prev, const float* mu, int64_t M, const void* g,
                                    void* gx, float* gmu, void* gprev, void* ws, size_t ws_bytes,
                                    hipStream_t stream);

/*
 * wkv_forward_gated: z = sigmoid(r) * WKV(w, u, k, v) elementwise, the gated
 * value the output projection W_o consumes, with the gate fused into the
 * output stores (one pass; no WKV intermediate in memory).  r and z are
 * [B, T, C] of dtype dt.  With `saved` non-NULL this is wkv_forward_save with
 * the gate (chunked algorithm, the states kept for the backward; workspace of
 * wkv_forward_workspace_bytes(..., WKV_ALGO_CHUNKED, 0)); with `saved` NULL the
 * algorithm is AUTO (workspace of wkv_forward_workspace_bytes(..., WKV_ALGO_AUTO,
 * 0)).  bfloat16 z: the float32 product of the float32 WKV output and the
 * gate, rounded to nearest even once.
 *
 * wkv_backward_gated: given gz = dL/dz, all of wkv_backward's gradients (for
 * dL/dy = gz * sigmoid(r)) and gr = dL/dr = gz * WKV * sigmoid(r) *
 * sigmoid(-r) ([B, T, C], dtype dt), in the same single backward scan.
 * `saved` as in wkv_backward_saved, or NULL to recompute the forward states;
 * workspace of wkv_backward_workspace_bytes(...).
 */
wkv_status wkv_forward_gated(int64_t B, int64_t T, int64_t C, wkv_dtype dt,
                             const float* w, const float* u,
                             const void* k, const void* v, const void* r, void* z,
                             float* saved, size_t saved_bytes,
                             void* ws, size_t ws_bytes, hipStream_t stream);

wkv_status wkv_backward_gated(int64_t B, int64_t T, int64_t C, wkv_dtype dt,
                              const float* w, const float* u,
                              const void* k, const void* v, const void* r, const void* gz,
                              const float* saved, size_t saved_bytes,
                              void* gk, void* gv, void* gr, float* gw, float* gu,
                              void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Causal linear attention, the second workload (page "Transformers are RNNs:
 * 선형 어텐션으로 만드는 빠른 자기회귀 트랜스포머", sections "인과 마스킹과 누적합" and
 * "특징 맵 선택과 계산 비용"): for every sequence b < BH (batch x heads) and
 * position i,
 *   out_i = sum_{j<=i} phi(q_i).phi(k_j) v_j / sum_{j<=i} phi(q_i).phi(k_j),
 * with phi(x) = elu(x) + 1 applied elementwise when feature_map is non-zero,
 * and q, k used as given (they must then be positive) when it is zero.
 *   q, k : [BH, N, D], v, out : [BH, N, M], dtype dt, dense row-major, each
 *        16-byte aligned (rows move with 16-byte accesses; WKV_EINVAL otherwise).
 * D and M may each be 32 or 64 (WKV_EINVAL otherwise).  float32
 * inputs use float32 matrix cores; bfloat16 inputs use bf16 matrix cores with
 * float32 accumulation (phi, the masked similarities and the carried state
 * are rounded to bf16 as operands).  Chunks of positions pass their states
 * along each sequence either by a decoupled look-back within one launch (q,
 * k, v read once, as in the chunked WKV forward) or through a separate scan
 * launch (see wkv_linear_attention_ex).
 *   ws : device workspace of at least wkv_linear_attention_workspace_bytes(...)
 *        bytes, zero-filled before its first use (wkv_forward_workspace_init)
 *        and then owned by the library between calls: it keeps a launch
 *        counter and per-chunk records (wkv_forward_workspace_query reports on
 *        it as on a forward workspace).  One workspace must not be used by two
 *        calls that may run at the same time.
 * Keys below about -87 underflow phi in float32.
 */
size_t wkv_linear_attention_workspace_bytes(int64_t BH, int64_t N, int64_t D, int64_t M,
                                            wkv_dtype dt);

wkv_status wkv_linear_attention(int64_t BH, int64_t N, int64_t D, int64_t M, wkv_dtype dt,
                                const void* q, const void* k, const void* v, void* out,
                                int feature_map, void* ws, size_t ws_bytes,
                                hipStream_t stream);

/*
 * wkv_linear_attention with the evaluation chosen: WKV_LA_ONE_PASS (one
 * launch, chunk states passed along each sequence by look-backs), or
 * WKV_LA_THREE_LAUNCHES (chunk aggregates, their prefix sums, outputs: q, k,
 * v are read in the first and third launches, but no chunk waits for
 * another, which is faster when few long sequences make the chain of
 * look-backs the longer path).  WKV_LA_AUTO picks by the sizes (what
 * wkv_linear_attention does).  Both give the same bits.  Another value gives
 * WKV_EINVAL.  The workspace size is the same for every choice.
 */
typedef enum { WKV_LA_AUTO = 0, WKV_LA_THREE_LAUNCHES = 1, WKV_LA_ONE_PASS = 2 } wkv_la_algo;

wkv_status wkv_linear_attention_ex(int64_t BH, int64_t N, int64_t D, int64_t M, wkv_dtype dt,
                                   const void* q, const void* k, const void* v, void* out,
                                   int feature_map, void* ws, size_t ws_bytes,
                                   wkv_la_algo algo, hipStream_t stream);

/*
 * One RNN-mode decoding step for N sequences x G layer slots x C channels
 * (section "RNN-유사추론" equation, and steps 4 and 7 of its decoding list:
 * update the WKV state, then store it for the next token).
 *   w, u    : [G, C] float32 device arrays (shared by the N sequences).
 *   k, v    : [N, G, C] device arrays of dtype dt (read only).
 *   a, b, p : [N, G, C] float32 device arrays: the state before the token on
 *             entry, the state after it on return (updated in place).
 *   y       : [N, G, C] device array of dtype dt (written).
 */
wkv_status wkv_step(int64_t N, int64_t G, int64_t C, wkv_dtype dt,
                    const float* w, const float* u,
                    const void* k, const void* v,
                    float* a, float* b, float* p,
                    void* y, hipStream_t stream);

/* A static, human-readable name for a status code. */
const char* wkv_status_string(wkv_status s);

#ifdef __cplusplus
}
#endif

#endif /* LIBWKV_H */
