// Internal interface between the C-ABI host code and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wkv {

// Control block at the start of a chunked workspace (zero-filled before first use).
// The ticket and done counters take every workgroup's atomic add, so each sits alone
// in its cache line: a plain read of a word sharing such a line queues behind the
// atomics and stalls the reading tile.
constexpr int kCtrlTicket = 0;   // tile ticket counter (zero between launches)
constexpr int kCtrlEpoch = 32;   // record epoch: number of completed launches, mod 2^30
constexpr int kCtrlForce = 40;   // launches still to run as if every wait gave up at once (set by the host)
constexpr int kCtrlGiveUp = 48;  // (epoch | kCtrlGiveUpMark) once a launch gave up waiting
constexpr int kCtrlDone = 64;    // workgroups finished in the current launch
constexpr int kCtrlWords = 128;  // 512 bytes
constexpr uint32_t kCtrlEpochMask = 0x3fffffffu;
constexpr uint32_t kCtrlGiveUpMark = 0x40000000u;

// Time steps per tile of the backward scan.
constexpr int kBwdTile = 128;

// Arguments of the forward kernels (plain pointers; see include/libwkv.h for meaning).
struct FwdArgs {
    const float* w;
    const float* u;
    const void* k;
    const void* v;
    void* y;
    const void* r;       // optional gate [B, T, C] dtype: y becomes sigmoid(r) * wkv (null: no gate)
    const float* sin_a;  // state in, [B, C] each, or all null for the empty state
    const float* sin_b;
    const float* sin_p;
    float* sout_a;  // state out, [B, C] each, or all null
    float* sout_b;
    float* sout_p;
    // chunked algorithm only (workspace carve-up)
    uint32_t* ctrl;  // control block, kCtrlWords words
    float* dump_a;     // optional [ceil(T / kBwdTile)][n_groups * 64] state entering every
    float* dump_b;     //   kBwdTile-th time step (record form: A = a 2^p, B = b 2^p, p in
    float* dump_p;     //   log2 units; needs tile >= kBwdTile); y may then be null (no outputs)
    uint32_t* status;  // [n_groups][n_chunks] status hints
    void* recs;        // [n_chunks][n_groups][2][3][64] tagged 64-bit words
    int B, T, C;
    int groups_per_row;  // ceil(C / 64)
    int n_groups;        // B * groups_per_row
    int n_chunks;        // ceil(T / tile)
    int by_index;        // 1: every tile of the launch can be resident at once, and tiles are
                         //   numbered by workgroup index instead of a ticket (chunked only)
};

// How the chunked kernel moves k, v, y (and r): float32 rows; bfloat16 rows at 2 bytes per
// lane; bfloat16 row pairs at 4 bytes per lane (even C, 4-byte aligned k, v, y, r).  Every mode
// runs one channel per lane, 64 channels per group.
enum IoMode { kIoF32 = 0, kIoBf16 = 1, kIoBf16Pair = 2 };

// io: an IoMode (below), as for the chunked kernel.
hipError_t launch_fwd_seq(const FwdArgs& a, int io, hipStream_t s);
// tile: 64, 128, 256 or 512 time steps per workgroup.
hipError_t launch_fwd_chunked(const FwdArgs& a, int io, int tile, hipStream_t s);
// Workgroups of the index-numbered chunked kernel one compute unit holds at once (0 if unknown).
int fwd_chunked_resident_per_cu(int io, int tile, bool gate);
hipError_t launch_zero_words(void* p, size_t n_words, hipStream_t s);
hipError_t launch_set_word(uint32_t* p, uint32_t value, hipStream_t s);
hipError_t launch_copy_state(const float* ia, const float* ib, const float* ip, float* oa,
                             float* ob, float* op, long n, hipStream_t s);

// Backward (gradients of sum(gy * y)): a chained scan backwards in time over tiles of
// kBwdTile tokens x 64 channels, started from the forward states the forward kernel dumped
// at those tiles' starts.
struct BwdArgs {
    const float* w;
    const float* u;
    const void* k;   // [B, T, C] dtype
    const void* v;
    const void* gy;  // dL/dy (dL/dz of the gated output z = sigmoid(r) y when r is set)
    const void* r;   // optional gate [B, T, C] dtype (null: no gate)
    void* gr;        // [B, T, C] dtype, dL/dr when r is set
    void* gk;        // [B, T, C] dtype
    void* gv;
    float* gw;       // [B, C] per-lane dL/dw, written by the reduction
    float* gu;
    const float* fw_a;  // [n_chunks][n_lanes] forward state entering each tile (dump)
    const float* fw_b;
    const float* fw_p;
    float* part;        // [2][n_chunks][n_lanes] per-tile dL/dw, dL/du partial sums
    long plane;         // float stride between the planes of fw_* and part (>= n_chunks * n_lanes)
    uint32_t* ctrl;     // control block (shared with the forward scan, which runs first)
    uint32_t* status;   // [n_groups][n_chunks] status hints
    void* rrecs;        // [n_chunks][n_groups][2][5][64] tagged 64-bit words
    bool inherit_give_up;  // a forward scan ran just before on the same control block
    int B, T, C;
    int groups_per_row, n_groups, n_chunks;
    long n_lanes;       // n_groups * 64
};
// io: IoMode of k, v, gy, gk, gv (row pairs need even C and 4-byte aligned arrays).
hipError_t launch_bwd(const BwdArgs& a, int io, hipStream_t s);

// Token shift: out[m] = mu[m] x_t + (1 - mu[m]) x_{t-1} for m < M (see wkv_mix.hip).
constexpr int kShiftMaxM = 4;
struct ShiftArgs {
    const void* x;       // [B, T, C] dtype
    const void* x_prev;  // [B, C] dtype, the token before the sequence, or null (zero)
    const float* mu;     // [M, C]
    void* out;           // [M, B, T, C] dtype
    int B, T, C, M;
};
// vec: 16-byte vectors of channels (C a multiple of 4 (f32) or 8 (bf16), 16-byte aligned x,
// x_prev, out); otherwise one element per thread.
hipError_t launch_token_shift(const ShiftArgs& a, int dtype, bool vec, hipStream_t s);

// Backward of the token shift (see wkv_mix.hip).
struct ShiftBwdArgs {
    const void* x;       // [B, T, C] dtype
    const void* x_prev;  // [B, C] dtype or null (zero)
    const float* mu;     // [M, C]
    const void* g;       // [M, B, T, C] dtype: dL/dout
    void* gx;            // [B, T, C] dtype
    float* gmu;          // [M, B, C] float32, per lane
    void* gprev;         // [B, C] dtype or null (not wanted)
    float* part;         // [n_seg][M][B][C] float32 partial sums (workspace)
    int B, T, C, M;
};
hipError_t launch_token_shift_backward(const ShiftBwdArgs& a, int dtype, int vec, hipStream_t s);
long token_shift_segments(long T);
hipError_t launch_zero_u16(void* p, long n, hipStream_t s);

// Causal linear attention (see la_forward.hip): q, k [BH, N, D], v, out [BH, N, M] of one dtype.
struct LaArgs {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    // one pass
    uint32_t* ctrl;    // control block, kCtrlWords words (the chunked forward's layout)
    uint32_t* status;  // [BH][n_chunks] status hints
    void* recs;        // [BH][n_chunks][2][D * M + D] tagged 64-bit words: aggregate, inclusive state
    // three launches
    float* agg;  // [BH][n_chunks][D * M + D] chunk aggregates, then their exclusive prefix
    int BH, N, D, M;
    int n_chunks;  // ceil(N / la_chunk_len(D, M, dtype))
    int feature;   // apply phi = elu + 1 to q and k
    int one_pass;  // one launch with look-backs, or three launches (aggregates, scan, outputs)
};
// Positions per chunk for these head sizes (D and M each 32 or 64 are built).
int la_chunk_len(int D, int M, int dtype);  // dtype 0 float32, 1 bfloat16
hipError_t launch_linear_attention(const LaArgs& a, int dtype, hipStream_t s);

struct StepArgs {
    const float* w;  // [G, C]
    const float* u;
    const void* k;  // [N, G, C]
    const void* v;
    float* a;  // [N, G, C], in place
    float* b;
    float* p;
    void* y;
    long n_lanes;  // N * G * C
    int GC;        // G * C
};

hipError_t launch_step(const StepArgs& a, int dtype, int nch, hipStream_t s);

}  // namespace wkv
