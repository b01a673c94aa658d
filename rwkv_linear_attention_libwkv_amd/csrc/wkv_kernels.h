// Internal interface between the C-ABI host code and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wkv {

// Control block at the start of a chunked workspace.  The ticket counter takes every
// workgroup's atomic add, so it sits alone in its cache line: a plain read of a word
// sharing that line queues behind the atomics and stalls the reading tile.
constexpr int kCtrlTicket = 0;   // tile ticket counter (reset per launch)
constexpr int kCtrlEpoch = 32;   // record epoch (bumped per launch), 128 bytes in
constexpr int kCtrlGiveUp = 48;  // look-back give-up flag (reset per launch)
constexpr int kCtrlWords = 64;   // 256 bytes

// Arguments of the forward kernels (plain pointers; see include/libwkv.h for meaning).
struct FwdArgs {
    const float* w;
    const float* u;
    const void* k;
    const void* v;
    void* y;
    const float* sin_a;  // state in, [B, C] each, or all null for the empty state
    const float* sin_b;
    const float* sin_p;
    float* sout_a;  // state out, [B, C] each, or all null
    float* sout_b;
    float* sout_p;
    // chunked algorithm only (workspace carve-up)
    uint32_t* ctrl;  // control block, kCtrlWords words (see below)
    float* chan_d;   // [C] e^{-w}, written by the prep kernel
    float* chan_eu;  // [C] e^{u}
    uint32_t* status;  // [n_groups][n_chunks] status hints
    void* recs;        // [n_chunks][n_groups][2][3][64 * NCH] tagged 64-bit words
    int B, T, C;
    int groups_per_row;  // ceil(C / (64 * NCH))
    int n_groups;        // B * groups_per_row
    int n_chunks;        // ceil(T / tile)
};

// dtype: 0 = float32, 1 = bfloat16.  nch: channels per thread (1, 2 or 4).
hipError_t launch_fwd_seq(const FwdArgs& a, int dtype, int nch, hipStream_t s);
hipError_t launch_fwd_chunked(const FwdArgs& a, int dtype, int nch, int tile, hipStream_t s);
hipError_t launch_zero_words(void* p, size_t n_words, hipStream_t s);
hipError_t launch_copy_state(const float* ia, const float* ib, const float* ip, float* oa,
                             float* ob, float* op, long n, hipStream_t s);

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
