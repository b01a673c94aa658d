// Batched RNN-mode WKV step for gfx950.
//
// Page "Reinventing RNNs for the Transformer Era: RWKV" (velog review), section
// "RNN-유사추론": WKV_t = (A_t + e^{u+k_t} v_t) / (B_t + e^{u+k_t}) with a per-layer,
// per-channel state; its autoregressive decoding list updates the WKV state (step 4)
// and stores (A_t, B_t) for the next token (step 7).  The state advances as
// A <- e^{-w} A + e^{k} v, B <- e^{-w} B + e^{k} (the reading that reproduces the WKV
// equation).
//
// One thread owns NCH consecutive lanes (n, g, c); every byte is touched once, so the
// kernel streams k, v (read), the state a, b, p (read and written in place) and y
// (written): 30 bytes per lane for bfloat16 k, v, y.  Exponents are formed in float64
// and the new float32 reference p is chosen first, so the stored (a, b) carry the
// exact factor between the old and the new reference.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wkv_device.h"
#include "wkv_kernels.h"

namespace wkv {

// Every array except w and u is touched once per step: those accesses are non-temporal
// (nt), so they do not evict w and u (shared by the N sequences) from the caches.
typedef float vf32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int vu32x2 __attribute__((ext_vector_type(2)));

template <int NCH>
__device__ __forceinline__ void ld4(const float* __restrict__ p, float (&o)[NCH]) {
    if constexpr (NCH == 4) {
        const float4 t = *reinterpret_cast<const float4*>(p);
        o[0] = t.x; o[1] = t.y; o[2] = t.z; o[3] = t.w;
    } else {
#pragma unroll
        for (int i = 0; i < NCH; ++i) o[i] = p[i];
    }
}

template <int NCH>
__device__ __forceinline__ void ld4_nt(const float* __restrict__ p, float (&o)[NCH]) {
    if constexpr (NCH == 4) {
        const vf32x4 t = __builtin_nontemporal_load(reinterpret_cast<const vf32x4*>(p));
        o[0] = t.x; o[1] = t.y; o[2] = t.z; o[3] = t.w;
    } else {
#pragma unroll
        for (int i = 0; i < NCH; ++i) o[i] = __builtin_nontemporal_load(p + i);
    }
}

template <int NCH>
__device__ __forceinline__ void st4_nt(float* __restrict__ p, const float (&o)[NCH]) {
    if constexpr (NCH == 4) {
        const vf32x4 t = {o[0], o[1], o[2], o[3]};
        __builtin_nontemporal_store(t, reinterpret_cast<vf32x4*>(p));
    } else {
#pragma unroll
        for (int i = 0; i < NCH; ++i) __builtin_nontemporal_store(o[i], p + i);
    }
}

template <int NCH>
__device__ __forceinline__ void ld_io(const float* __restrict__ p, float (&o)[NCH]) { ld4_nt<NCH>(p, o); }

template <int NCH>
__device__ __forceinline__ void ld_io(const uint16_t* __restrict__ p, float (&o)[NCH]) {
    if constexpr (NCH == 4) {
        const vu32x2 t = __builtin_nontemporal_load(reinterpret_cast<const vu32x2*>(p));
        o[0] = __uint_as_float(t.x << 16);
        o[1] = __uint_as_float(t.x & 0xffff0000u);
        o[2] = __uint_as_float(t.y << 16);
        o[3] = __uint_as_float(t.y & 0xffff0000u);
    } else {
#pragma unroll
        for (int i = 0; i < NCH; ++i) o[i] = __uint_as_float((uint32_t)__builtin_nontemporal_load(p + i) << 16);
    }
}

template <int NCH>
__device__ __forceinline__ void st_io(float* __restrict__ p, const float (&o)[NCH]) { st4_nt<NCH>(p, o); }

typedef float sf32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 sbf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
    sf32x2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, sbf16x2));
}

template <int NCH>
__device__ __forceinline__ void st_io(uint16_t* __restrict__ p, const float (&o)[NCH]) {
    if constexpr (NCH == 4) {
        const vu32x2 t = {pack2_bf16(o[0], o[1]), pack2_bf16(o[2], o[3])};
        __builtin_nontemporal_store(t, reinterpret_cast<vu32x2*>(p));
    } else {
#pragma unroll
        for (int i = 0; i < NCH; ++i)
            __builtin_nontemporal_store((uint16_t)(pack2_bf16(o[i], 0.f) & 0xffffu), p + i);
    }
}

template <typename IO, int NCH>
__global__ __launch_bounds__(256) void step_kernel(StepArgs args) {
    const long gid = (long)blockIdx.x * 256 + threadIdx.x;
    const long li = gid * NCH;
    if (li >= args.n_lanes) return;
    const long wi = li % args.GC;

    float w[NCH], u[NCH], k[NCH], v[NCH], a[NCH], b[NCH], p[NCH], y[NCH];
    ld4<NCH>(args.w + wi, w);
    ld4<NCH>(args.u + wi, u);
    ld_io<NCH>(static_cast<const IO*>(args.k) + li, k);
    ld_io<NCH>(static_cast<const IO*>(args.v) + li, v);
    ld4_nt<NCH>(args.a + li, a);
    ld4_nt<NCH>(args.b + li, b);
    ld4_nt<NCH>(args.p + li, p);

#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const double p2 = (double)p[i] * kLog2eD;
        const double k2 = (double)k[i] * kLog2eD;
        // output: (A + e^{u+k} v) / (B + e^{u+k})
        const double uk = (double)u[i] * kLog2eD + k2;
        const double q = fmax(p2, uk);
        const float e1 = ex2((float)(p2 - q));
        const float e2 = ex2((float)(uk - q));
        y[i] = fmaf(e1, a[i], e2 * v[i]) * rcp(fmaf(e1, b[i], e2));
        // update: A <- e^{-w} A + e^{k} v, B <- e^{-w} B + e^{k}
        const double pw = p2 - (double)w[i] * kLog2eD;
        const double q2 = fmax(pw, k2);
        const float pn = fmaxf((float)(q2 * kLn2D), kEmptyPf);  // new reference, natural log
        const double qr = (double)pn * kLog2eD;
        const float f1 = ex2((float)(pw - qr));
        const float f2 = ex2((float)(k2 - qr));
        a[i] = fmaf(f1, a[i], f2 * v[i]);
        b[i] = fmaf(f1, b[i], f2);
        p[i] = pn;
    }
    st_io<NCH>(static_cast<IO*>(args.y) + li, y);
    st4_nt<NCH>(args.a + li, a);
    st4_nt<NCH>(args.b + li, b);
    st4_nt<NCH>(args.p + li, p);
}

template <typename IO, int NCH>
static hipError_t launch_step_t(const StepArgs& a, hipStream_t s) {
    const long threads = a.n_lanes / NCH;
    const long blocks = (threads + 255) / 256;
    hipLaunchKernelGGL((step_kernel<IO, NCH>), dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_step(const StepArgs& a, int dtype, int nch, hipStream_t s) {
    if (dtype == 0) return nch == 4 ? launch_step_t<float, 4>(a, s) : launch_step_t<float, 1>(a, s);
    return nch == 4 ? launch_step_t<uint16_t, 4>(a, s) : launch_step_t<uint16_t, 1>(a, s);
}

}  // namespace wkv
