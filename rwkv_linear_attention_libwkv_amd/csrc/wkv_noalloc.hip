// wkv_forward_noalloc: wkv_forward with its workspace in a static device array, for callers
// that cannot allocate (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  Same kernels and results as wkv_forward with a workspace of the same
// size; nothing here allocates.
//
// The array `scratch` exists once per GPU the library runs on and lives until the process
// ends.  Host code never uses its name as an address (in host code the name is a host-side
// stand-in, not device memory): the first call on a device, with that device current, looks
// up the device address with hipGetSymbolAddress and keeps it per device; every later use
// (kernel arguments) goes through that pointer.
//
// Contents.  The chunked scan keeps its launch counters and per-tile records in the array
// between calls (records carry the launch epoch, so old ones are never mistaken for new).
// The array is zero at load; the first call on a device also zero-fills the two counters a
// launch must find at zero, leaving the epoch, and every launch's last workgroup resets them
// for the next.  Calls on one GPU share its array: two calls that may overlap in time on the
// same GPU (different streams, or different host threads) race and must not be made.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "libwkv.h"
#include "wkv_kernels.h"

namespace {

// 32 MiB: the chunked workspace of up to about 10,900 tiles (a 65,536-token sequence of
// 5,120 bfloat16 channels needs 31.5 MB; 8 x 8,192 x 2,048 float32 needs 25 MB).
constexpr size_t kScratchBytes = (size_t)32 << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_setup_mutex;
void* g_scratch_ptr[kMaxDevices] = {};  // device address of `scratch` on each device, once looked up

// The device address of this device's array, looked up on first use (with the device current);
// the counters a launch must find at zero are cleared then, on `stream`, by a kernel.
wkv_status device_scratch(hipStream_t stream, void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return WKV_EHIP;
    std::lock_guard<std::mutex> lock(g_setup_mutex);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return WKV_EHIP;
        uint32_t* ctrl = static_cast<uint32_t*>(ptr);  // 256-aligned: the control block is at the start
        if (wkv::launch_set_word(ctrl + wkv::kCtrlTicket, 0u, stream) != hipSuccess ||
            wkv::launch_set_word(ctrl + wkv::kCtrlDone, 0u, stream) != hipSuccess ||
            wkv::launch_set_word(ctrl + wkv::kCtrlForce, 0u, stream) != hipSuccess)
            return WKV_EHIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return WKV_OK;
}

}  // namespace

extern "C" wkv_status wkv_forward_noalloc(int64_t B, int64_t T, int64_t C, wkv_dtype dt, const float* w,
                                          const float* u, const void* k, const void* v, void* y,
                                          hipStream_t stream) {
    const size_t need = wkv_forward_workspace_bytes(B, T, C, dt, WKV_ALGO_AUTO, 0);
    if (need == (size_t)-1) return dt == WKV_F32 || dt == WKV_BF16 ? WKV_EINVAL : WKV_EDTYPE;
    if (need > kScratchBytes) {
        // beyond the array: the sequential algorithm, which needs no workspace, when its grid
        // can hold the batch rows
        if (B > 65535) return WKV_EWORKSPACE;
        return wkv_forward_ex(B, T, C, dt, w, u, k, v, y, nullptr, 0, WKV_ALGO_SEQ, 0, stream);
    }
    if (need == 0)  // empty problem or sequential algorithm: no workspace at all
        return wkv_forward(B, T, C, dt, w, u, k, v, y, nullptr, 0, stream);
    if (!w || !u || !k || !v || !y) return WKV_EINVAL;
    void* ws = nullptr;
    const wkv_status st = device_scratch(stream, &ws);
    if (st != WKV_OK) return st;
    return wkv_forward(B, T, C, dt, w, u, k, v, y, ws, kScratchBytes, stream);
}
