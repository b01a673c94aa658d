// Device arithmetic of the WKV recurrence for gfx950 (shared by the forward kernels).
//
// Operator: page "Reinventing RNNs for the Transformer Era: RWKV" (velog review),
// section "WKV 연산자", WKV equation; RNN form in section "RNN-유사추론".
// Per channel the state (A, B) advances as A <- e^{-w} A + e^{k} v, B <- e^{-w} B + e^{k},
// and the output of a token is (A + e^{u+k} v) / (B + e^{u+k}).
//
// Representation.  Inside the kernels a state is a Carry {a, b, p} meaning
// A = a * 2^p, B = b * 2^p with p a float64 exponent in log2 units.  Keeping p in
// float64 and applying decays multiplicatively means no exponent is ever rounded
// to float32 and re-used: p only selects a reference, and every factor between
// two references is 2^(difference) with the difference formed in float64.
//
// Chunk fast path (used when the exponents of a chunk are well conditioned).
// For L consecutive tokens and a reference R = max_j k_j (log2 units):
//   x_j   = 2^(k_j log2e - R)                 (one exp per token, x_j <= 1)
//   A/2^R <- d * A/2^R + x_j v_j,  d = e^{-w}  (d is a per-channel constant)
//   y_j   = (A/2^R + e^u x_j v_j) / (B/2^R + e^u x_j)
// so a token costs one exp and one reciprocal.  The path is taken only when
// every exponent of the chunk lies within kSpan (log2 units) of R, so that no
// term that matters can underflow and none can overflow; otherwise the chunk
// runs the exact per-token log-sum-exp update (the fallback below).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wkv {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr double kLog2eD = 1.4426950408889634073599;
constexpr double kLn2D = 0.6931471805599453094172;
// exponent (log2 units) of the empty state; finite so that differences never give inf - inf
constexpr double kEmptyP = -1.0e300;
// smallest p a stored float32 state may carry (the ABI's WKV_P_EMPTY is -1e38 natural log)
constexpr float kEmptyPf = -1.0e38f;
// fast path: maximum spread, in log2 units, between the chunk reference and any exponent
constexpr float kSpan = 60.0f;

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }

struct Carry {
    float a, b;
    double p;
};

__device__ __forceinline__ Carry empty_carry() { return {0.f, 0.f, kEmptyP}; }

// X followed by Y, where Y spans `decay` = (number of tokens in Y) * w * log2e.
// A_{X then Y} = e^{-n_Y w} A_X + A_Y, and the same for B.
__device__ __forceinline__ Carry combine(const Carry& x, const Carry& y, double decay) {
    const double px = x.p - decay;
    const double pm = fmax(px, y.p);
    const float fx = ex2((float)(px - pm));
    const float fy = ex2((float)(y.p - pm));
    return {fmaf(x.a, fx, y.a * fy), fmaf(x.b, fx, y.b * fy), pm};
}

// Same state with b scaled into [0.5, 1) by an exact power of two.
__device__ __forceinline__ Carry normalize(const Carry& c) {
    int e;
    const float m = __builtin_frexpf(c.b, &e);
    return {__builtin_ldexpf(c.a, -e), m, c.p + (double)e};
}

// Per-channel constants, computed once per channel per kernel.
struct Chan {
    float d;   // e^{-w}
    float eu;  // e^{u}
    float w;   // decay rate
    float u;   // bonus
};

__device__ __forceinline__ Chan make_chan(float w, float u) {
    return Chan{(float)exp(-(double)w), (float)exp((double)u), w, u};
}
__device__ __forceinline__ double w2_of(const Chan& c) { return (double)c.w * kLog2eD; }
__device__ __forceinline__ double u2_of(const Chan& c) { return (double)c.u * kLog2eD; }

// Channel constants allow the fast path: w >= 0 (decay, so d <= 1) and |u| log2e <= kSpan.
__device__ __forceinline__ bool chan_fast_ok(const Chan& c) {
    const float u2 = c.u * kLog2e;
    return (c.w >= 0.f) && (c.w <= 3.0e38f) && (u2 <= kSpan) && (u2 >= -kSpan);
}

// Fast-path conditions of a chunk: channel constants, the key range and the bonus stay
// within kSpan of the reference R = max k (log2 units).
__device__ __forceinline__ bool chunk_fast_ok(const Chan& ch, float kmax, float kmin) {
    const float range = (kmax - kmin) * kLog2e;
    return chan_fast_ok(ch) && (range <= kSpan) && (range - ch.u * kLog2e <= kSpan);
}

// float32 -> float32 state triple of the ABI (natural-log p) from a Carry.
__device__ __forceinline__ void carry_to_abi(const Carry& c, float& a, float& b, float& p) {
    if (c.b == 0.f && c.a == 0.f) {  // empty
        a = 0.f;
        b = 0.f;
        p = kEmptyPf;
        return;
    }
    const double pn = c.p * kLn2D;
    float pf = (float)pn;
    pf = fmaxf(pf, kEmptyPf);
    const float r = ex2((float)(c.p - (double)pf * kLog2eD));
    a = c.a * r;
    b = c.b * r;
    p = pf;
}

// Carry from the ABI's state triple.
__device__ __forceinline__ Carry carry_from_abi(float a, float b, float p) {
    return normalize(Carry{a, b, (double)p * kLog2eD});
}

}  // namespace wkv
