// Row loads and stores and the exact per-token recurrence, shared by the forward and
// backward kernels for gfx950.  See wkv_device.h for the state representation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "wkv_device.h"

namespace wkv {

// ----------------------------------------------------------------------------
// Row loads and stores: one channel per lane of one time step.
//
// A wave addresses its rows through a buffer resource whose base is wave-uniform
// (scalar registers), a per-lane 32-bit byte offset (one VGPR for all rows) and a
// per-row scalar offset, so a chunk of rows costs no per-row address registers.
// ----------------------------------------------------------------------------

typedef __amdgpu_buffer_rsrc_t Rsrc;

__device__ __forceinline__ Rsrc make_rsrc(const void* base) {
    // raw buffer (stride 0), 2^31-1 addressable bytes, gfx9 data-format word
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
}

// Cache policy of the k, v loads and y stores: non-temporal (nt).  Every element is
// touched once, so keeping these lines in L2 and the MALL only evicts the look-back
// records that are reused; measured 6.1 TB/s for a plain 12-byte-per-element stream
// with nt against 5.7 TB/s without.
constexpr int kStream = 2;

__device__ __forceinline__ float bf_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// float32 pair -> packed bfloat16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    f32x2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// bfloat16 rows read and written two rows at a time: lanes 0-31 move channels (2i, 2i+1)
// of row r and lanes 32-63 the same channels of row r+1, four bytes per lane; trading
// words with the partner lane (lane ^ 32) then gives every lane both rows of a single
// channel, lane i < 32 owning channel 2i and lane 32+i channel 2i+1.  A wave thus covers
// 64 channels with 4-byte accesses and one channel per lane.  Needs an even C and
// 4-byte aligned k, v, y.
struct Bf16Pair {
    uint16_t bits;
};
template <typename IO>
constexpr bool kPair = std::is_same<IO, Bf16Pair>::value;

// channel (within the wave's 64) of a lane in row-pair mode
__device__ __forceinline__ int pair_channel(int lane) { return ((lane & 31) << 1) | (lane >> 5); }

// Row-pair exchange, the same operation in both directions.  Load: x is the lane's word
// of its row (channels 2i, 2i+1); the result holds the lane's own channel in rows r
// (low half) and r+1 (high half).  Store: x holds the lane's own channel in rows r, r+1;
// the result is the lane's word of its row.  The partner's word comes through
// ds_bpermute (one result register, unlike a two-register swap, which kept twice the
// in-flight words alive); v_perm_b32 then picks the halves: lanes 0-31 the low halves
// (own word first), lanes 32-63 the high halves (partner's word first).
__device__ __forceinline__ uint32_t pair_exchange(uint32_t x, uint32_t partner_addr, uint32_t sel) {
    const uint32_t other = (uint32_t)__builtin_amdgcn_ds_bpermute((int)partner_addr, (int)x);
    return __builtin_amdgcn_perm(other, x, sel);
}
__device__ __forceinline__ uint32_t pair_sel(uint32_t upper) { return upper ? 0x03020706u : 0x05040100u; }

// One time step of this lane's channel (2-byte or 4-byte element).
template <typename IO>
__device__ __forceinline__ float load_elt(Rsrc r, uint32_t voff, uint32_t soff) {
    if constexpr (sizeof(IO) == 4)
        return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kStream));
    else
        return bf_lo((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, kStream));
}

template <typename IO>
__device__ __forceinline__ void store_elt(Rsrc r, uint32_t voff, uint32_t soff, float y) {
    if constexpr (sizeof(IO) == 4)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y), r, voff, soff, kStream);
    else
        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(pack_bf16(y, 0.f) & 0xffffu), r, voff,
                                              soff, kStream);
}

// The rows of one wave: k, v, y resources based at the wave's first row and first channel.
struct WaveRows {
    Rsrc k, v, y;
    Rsrc r;              // gate rows when the output is sigmoid(r) * wkv (unused otherwise)
    uint32_t lane_off;   // byte offset of this lane's channel within a row
    uint32_t row_bytes;  // C * element size
    uint32_t pair_off;   // row-pair mode: byte offset of this lane's 4-byte word in a row pair
    uint32_t upper;      // row-pair mode: 1 for lanes 32-63 (the second row of a pair)
    uint32_t partner;    // row-pair mode: ds_bpermute address of lane ^ 32
};

// ----------------------------------------------------------------------------
// Per-token arithmetic.
// ----------------------------------------------------------------------------

// Logistic sigmoid 1 / (1 + e^{-r}) (the output gate): saturates to 0 and 1 without NaN.
__device__ __forceinline__ float sigmoid_f(float r) { return rcp(1.f + ex2(-r * kLog2e)); }

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

// Exact walk over the wave's first n rows read from memory, advancing c; writes y rows
// (sigmoid(r) * y rows when GATE) when OUT and `store`.  Rolled loop: this path is rare
// and keeps no chunk in registers.
template <typename IO, bool OUT, bool GATE = false>
__device__ __forceinline__ void lse_walk(const Chan& ch, Carry& c, const WaveRows& w, int n, bool load,
                                         bool store) {
#pragma unroll 1
    for (int j = 0; j < n; ++j) {
        const uint32_t so = (uint32_t)j * w.row_bytes;
        const float k = load ? load_elt<IO>(w.k, w.lane_off, so) : 0.f;
        const float v = load ? load_elt<IO>(w.v, w.lane_off, so) : 0.f;
        float y = lse_token<OUT>(ch, c, k, v);
        if constexpr (GATE) y *= sigmoid_f(load ? load_elt<IO>(w.r, w.lane_off, so) : 0.f);
        if (OUT && store) store_elt<IO>(w.y, w.lane_off, so, y);
    }
}

// Exact walk over n rows of one lane's channel read from memory (no outputs), advancing c:
// rows k_base + j * row_bytes (and v alike) at byte offset lane_off, four rows loaded
// together, the resource rebased every four rows so any n stays within its range.  Lanes
// with !valid read zeros.  Small on purpose: it runs only on the give-up path, and its
// registers count against the whole kernel.
template <typename IO>
__device__ __forceinline__ void walk_rows_exact(const Chan& ch, Carry& c, const char* k_base, const char* v_base,
                                                uint32_t lane_off, uint32_t row_bytes, int n, bool valid) {
    constexpr int kB = 4;
#pragma unroll 1
    for (int j0 = 0; j0 < n; j0 += kB) {
        const Rsrc rk = make_rsrc(k_base + (size_t)j0 * row_bytes);
        const Rsrc rv = make_rsrc(v_base + (size_t)j0 * row_bytes);
        float kk[kB], vv[kB];
#pragma unroll
        for (int j = 0; j < kB; ++j) {
            const bool in = valid && j0 + j < n;
            kk[j] = in ? load_elt<IO>(rk, lane_off, (uint32_t)j * row_bytes) : 0.f;
            vv[j] = in ? load_elt<IO>(rv, lane_off, (uint32_t)j * row_bytes) : 0.f;
        }
#pragma unroll 1
        for (int j = 0; j < kB; ++j)
            if (j0 + j < n) (void)lse_token<false>(ch, c, kk[j], vv[j]);
    }
}

}  // namespace wkv
