// libwkv C ABI: argument checks, algorithm and tile planning, workspace carve-up and
// launches on the caller's stream.  Every check runs before any HIP call; nothing here
// allocates or keeps state between calls, and only the workspace query synchronises.
#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <climits>

#include "libwkv.h"
#include "wkv_kernels.h"

namespace {

constexpr size_t kAlign = 256;
constexpr int kDefaultTile = 256;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool dtype_ok(wkv_dtype dt) { return dt == WKV_F32 || dt == WKV_BF16; }
size_t dtype_size(wkv_dtype dt) { return dt == WKV_F32 ? 4 : 2; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// The chunked kernel moves bfloat16 rows two at a time (4 bytes per lane) when C is even
// and k, v, y are 4-byte aligned; 2-byte lanes otherwise.
int chunk_io(wkv_dtype dt, int64_t C, const void* k, const void* v, const void* y) {
    if (dt == WKV_F32) return wkv::kIoF32;
    const bool pairs = C % 2 == 0 && aligned(k, 4) && aligned(v, 4) && aligned(y, 4);
    return pairs ? wkv::kIoBf16Pair : wkv::kIoBf16;
}

bool tile_ok(int64_t t) { return t == 0 || t == 64 || t == 128 || t == 256 || t == 512; }

// AUTO: the chunked scan, except for sequences of at most 64 tokens (too short to fill a
// tile's waves), which walk T sequentially.  Measured on MI355X (interleaved, per call): the
// chunked scan also wins where every (b, c) lane has a thread of its own, float32 B=4096 T=128
// C=768 826 against 890 us, B=2048 T=256 C=1024 1001 against 1187 us, B=1024 T=2048 C=512 2144
// against 2349 us, bf16 B=256 T=2048 C=2048 1192 against 2342 us; at T=64 (B=8192, C=1024
// float32) the sequential kernel wins, 1134 against 1745 us.
int resolve_algo(wkv_algo algo, int64_t B, int64_t T, int64_t C) {
    if (algo != WKV_ALGO_AUTO) return (int)algo;
    (void)C;
    if (B > 65535) return WKV_ALGO_CHUNKED;  // the sequential grid holds batch rows in y
    return T <= 64 ? WKV_ALGO_SEQ : WKV_ALGO_CHUNKED;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Compute units of the current device (0 if unknown), looked up once per device.
int cu_count() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0 && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
        cached[dev].store(n, std::memory_order_relaxed);
    return n > 0 ? n : 0;
}

// Chunk length when the caller passes 0: 256, or 512 for problems of fewer than 1024
// tiles of 256, where the per-tile look-back dominates (B=8, T=1024, C=768 float32:
// 20 us at 512 against 25 us at 256).
int default_tile(int64_t B, int64_t T, int64_t C) {
    const int64_t tiles = B * ceil_div(C, 64) * ceil_div(T, kDefaultTile);
    return tiles < 1024 ? 2 * kDefaultTile : kDefaultTile;
}

// Workspace of the chunked algorithm: [control words][status word per tile][records: per
// tile and channel, two states of three tagged 64-bit words].
struct ChunkLayout {
    size_t off_status, off_recs, total;
};

ChunkLayout chunked_layout(int64_t B, int64_t T, int64_t C, int tile) {
    const int64_t n_groups = B * ceil_div(C, 64);
    const int64_t n_tiles = n_groups * ceil_div(T, tile);
    ChunkLayout L;
    L.off_status = align_up((size_t)wkv::kCtrlWords * 4, kAlign);
    L.off_recs = L.off_status + align_up((size_t)n_tiles * 4, kAlign);
    L.total = L.off_recs + (size_t)n_tiles * 2 * 3 * 64 * 8 + kAlign;  // + slack to align the base
    return L;
}

size_t chunked_bytes_bound(int64_t B, int64_t T, int64_t C, int tile) { return chunked_layout(B, T, C, tile).total; }

bool sizes_ok(int64_t B, int64_t T, int64_t C) {
    if (B < 0 || T < 0 || C < 0) return false;
    if (B > INT_MAX || T > INT_MAX || C > INT_MAX) return false;
    if (B > 0 && C > 0 && B * C > INT_MAX) return false;
    return true;
}

// The scan kernels address a wave's rows through one buffer resource (2^31 - 1 bytes) with
// 32-bit row offsets, up to kMaxRowsPerRsrc rows from its base: rows of C elements must keep
// that window addressable.
constexpr int64_t kMaxRowsPerRsrc = 64;
bool rows_ok(int64_t C, wkv_dtype dt) { return C * (int64_t)dtype_size(dt) * kMaxRowsPerRsrc <= (int64_t)INT_MAX; }

// States saved for the backward: 3 float32 planes (a, b, p in record form) of
// [ceil(T / kBwdTile)][n_lanes], each plane padded to kAlign bytes.
size_t saved_plane_bytes(int64_t B, int64_t T, int64_t C) {
    return align_up((size_t)ceil_div(T, wkv::kBwdTile) * (size_t)(B * ceil_div(C, 64) * 64) * 4, kAlign);
}

wkv_status forward_impl(int64_t B, int64_t T, int64_t C, wkv_dtype dt, const float* w,
                        const float* u, const void* k, const void* v, void* y,
                        const float* sia, const float* sib, const float* sip, float* soa,
                        float* sob, float* sop, void* ws, size_t ws_bytes, wkv_algo algo,
                        int64_t chunk_len, hipStream_t stream, float* saved = nullptr,
                        const void* r = nullptr) {
    if (!sizes_ok(B, T, C)) return WKV_EINVAL;
    if (!dtype_ok(dt)) return WKV_EDTYPE;
    if (!rows_ok(C, dt)) return WKV_EINVAL;
    if (algo != WKV_ALGO_AUTO && algo != WKV_ALGO_SEQ && algo != WKV_ALGO_CHUNKED) return WKV_EINVAL;
    if (!tile_ok(chunk_len)) return WKV_EINVAL;
    const bool in_any = sia || sib || sip, in_all = sia && sib && sip;
    const bool out_any = soa || sob || sop, out_all = soa && sob && sop;
    if (in_any != in_all || out_any != out_all) return WKV_EINVAL;
    if (B == 0 || C == 0) return WKV_OK;
    if (T == 0) {
        if (!out_all) return WKV_OK;
        if (soa == sia && sob == sib && sop == sip) return WKV_OK;
        return wkv::launch_copy_state(sia, sib, sip, soa, sob, sop, (long)(B * C), stream) == hipSuccess
                   ? WKV_OK
                   : WKV_EHIP;
    }
    if (!w || !u || !k || !v || !y) return WKV_EINVAL;

    wkv::FwdArgs a{};
    a.w = w;
    a.u = u;
    a.k = k;
    a.v = v;
    a.y = y;
    a.r = r;
    a.sin_a = sia;
    a.sin_b = sib;
    a.sin_p = sip;
    a.sout_a = soa;
    a.sout_b = sob;
    a.sout_p = sop;
    a.B = (int)B;
    a.T = (int)T;
    a.C = (int)C;

    const int resolved = resolve_algo(algo, B, T, C);
    int io = chunk_io(dt, C, k, v, y);
    if (io == wkv::kIoBf16Pair && r && !aligned(r, 4)) io = wkv::kIoBf16;
    if (resolved == WKV_ALGO_SEQ) {
        if (B > 65535) return WKV_EINVAL;  // batch rows are grid.y
        return wkv::launch_fwd_seq(a, io, stream) == hipSuccess ? WKV_OK : WKV_EHIP;
    }

    // bfloat16 row pairs hold 64 tokens per wave, so their tile of eight waves is 512 tokens
    // (B=1, T=65536, C=5120: 406-412 us against 414-418 us at 256; B=8, T=8192, C=2048:
    // 164-168 us against 170-172 us); it needs no more workspace than default_tile's
    const int tile = chunk_len ? (int)chunk_len : (io == wkv::kIoBf16Pair ? 2 * kDefaultTile : default_tile(B, T, C));
    if (saved && tile < wkv::kBwdTile) return WKV_EINVAL;
    const size_t need = chunked_bytes_bound(B, T, C, tile);
    if (!ws || ws_bytes < need) return WKV_EWORKSPACE;
    a.groups_per_row = (int)ceil_div(C, 64);
    a.n_groups = (int)(B * a.groups_per_row);
    a.n_chunks = (int)ceil_div(T, tile);
    const int64_t n_tiles = (int64_t)a.n_groups * a.n_chunks;
    if (n_tiles > INT_MAX) return WKV_EINVAL;
    // a launch whose tiles can all be resident at once numbers them by workgroup index (B=8,
    // T=1024, C=768 float32: 192 tiles, whose tickets would queue on one counter)
    a.by_index = n_tiles <= (int64_t)cu_count() * wkv::fwd_chunked_resident_per_cu(io, tile, r != nullptr) ? 1 : 0;
    const ChunkLayout L = chunked_layout(B, T, C, tile);
    char* base = reinterpret_cast<char*>(align_up(reinterpret_cast<uintptr_t>(ws), kAlign));
    a.ctrl = reinterpret_cast<uint32_t*>(base);
    a.status = reinterpret_cast<uint32_t*>(base + L.off_status);
    a.recs = base + L.off_recs;
    if (saved) {
        const size_t ps = saved_plane_bytes(B, T, C) / 4;
        a.dump_a = saved;
        a.dump_b = saved + ps;
        a.dump_p = saved + 2 * ps;
    }
    return wkv::launch_fwd_chunked(a, io, tile, stream) == hipSuccess ? WKV_OK : WKV_EHIP;
}

// Workspace of the backward: the forward chunked workspace at the forward's default tile
// (its control block first, so the forward diagnostics read it too; the backward scan
// reuses the control block after the forward scan), the backward scan's status words and
// records (two carries of five tagged 64-bit words per kBwdTile tile and channel), then
// float32 planes of [n_chunks][n_lanes]: 2 for partial sums, 3 for the forward states
// entering each tile (unused when the caller passes saved states).
constexpr int kBwdPlanes = 2 + 3;

struct BwdLayout {
    int fwd_tile;
    ChunkLayout fwd;
    size_t off_status, off_rrecs, off_planes, plane_bytes, total;
};

BwdLayout backward_layout(int64_t B, int64_t T, int64_t C) {
    BwdLayout L;
    L.fwd_tile = default_tile(B, T, C);
    L.fwd = chunked_layout(B, T, C, L.fwd_tile);
    const int64_t n_lanes = B * ceil_div(C, 64) * 64;
    const int64_t n_chunks = ceil_div(T, wkv::kBwdTile);
    const size_t n_tiles = (size_t)(n_lanes / 64) * (size_t)n_chunks;
    L.off_status = align_up(L.fwd.total, kAlign);
    L.off_rrecs = L.off_status + align_up(n_tiles * 4, kAlign);
    L.off_planes = L.off_rrecs + align_up(n_tiles * 2 * 5 * 64 * 8, kAlign);
    L.plane_bytes = align_up((size_t)n_chunks * (size_t)n_lanes * 4, kAlign);
    L.total = L.off_planes + kBwdPlanes * L.plane_bytes;
    return L;
}

// saved: states from wkv_forward_save, or null to recompute them with a forward scan.
// r, gr: the output gate and its gradient (both null without a gate; gy is then dL/dz).
wkv_status backward_impl(int64_t B, int64_t T, int64_t C, wkv_dtype dt, const float* w, const float* u,
                         const void* k, const void* v, const void* gy, const float* saved, size_t saved_bytes,
                         void* gk, void* gv, float* gw, float* gu, void* ws, size_t ws_bytes,
                         hipStream_t stream, const void* r = nullptr, void* gr = nullptr) {
    if (!sizes_ok(B, T, C)) return WKV_EINVAL;
    if (!dtype_ok(dt)) return WKV_EDTYPE;
    if (!rows_ok(C, dt)) return WKV_EINVAL;
    if (B == 0 || C == 0) return WKV_OK;
    if (!gw || !gu) return WKV_EINVAL;
    if (T == 0) {  // no token: every gradient of w and u is zero
        return wkv::launch_zero_words(gw, (size_t)(B * C), stream) == hipSuccess &&
                       wkv::launch_zero_words(gu, (size_t)(B * C), stream) == hipSuccess
                   ? WKV_OK
                   : WKV_EHIP;
    }
    if (!w || !u || !k || !v || !gy || !gk || !gv) return WKV_EINVAL;
    const size_t sps = saved_plane_bytes(B, T, C);
    if (saved && saved_bytes < 3 * sps) return WKV_EINVAL;
    const BwdLayout L = backward_layout(B, T, C);
    if (!ws || ws_bytes < L.total) return WKV_EWORKSPACE;
    const int groups_per_row = (int)ceil_div(C, 64);
    const int64_t n_groups = B * groups_per_row;
    const int64_t n_chunks = ceil_div(T, wkv::kBwdTile);
    if (n_groups * n_chunks > INT_MAX) return WKV_EINVAL;
    // ws is at least 4-byte aligned by the caller's allocator; the layout aligns every part
    char* base = reinterpret_cast<char*>(align_up(reinterpret_cast<uintptr_t>(ws), kAlign));
    float* planes = reinterpret_cast<float*>(base + L.off_planes);
    const size_t ps = L.plane_bytes / 4;  // plane stride in floats

    // 1. forward states entering every tile (no outputs), unless the caller saved them
    const float* fw = saved;
    size_t fps = sps / 4;
    uint32_t* ctrl = reinterpret_cast<uint32_t*>(base);
    if (!saved) {
        // the forward's own tile: 512 for bfloat16 row pairs (eight waves of 64 tokens), else the
        // default; its carve-up fits in the part of the workspace sized at the default tile
        const int io_f = chunk_io(dt, C, k, v, k);
        const int ftile = io_f == wkv::kIoBf16Pair ? 2 * kDefaultTile : L.fwd_tile;
        const ChunkLayout FL = chunked_layout(B, T, C, ftile);
        wkv::FwdArgs f{};
        f.w = w;
        f.u = u;
        f.k = k;
        f.v = v;
        f.y = nullptr;
        f.B = (int)B;
        f.T = (int)T;
        f.C = (int)C;
        f.groups_per_row = groups_per_row;
        f.n_groups = (int)n_groups;
        f.n_chunks = (int)ceil_div(T, ftile);
        f.by_index = n_groups * f.n_chunks <= (int64_t)cu_count() * wkv::fwd_chunked_resident_per_cu(io_f, ftile, false)
                         ? 1
                         : 0;
        f.ctrl = ctrl;
        f.status = reinterpret_cast<uint32_t*>(base + FL.off_status);
        f.recs = base + FL.off_recs;
        f.dump_a = planes + 2 * ps;
        f.dump_b = planes + 3 * ps;
        f.dump_p = planes + 4 * ps;
        if (wkv::launch_fwd_chunked(f, io_f, ftile, stream) != hipSuccess) return WKV_EHIP;
        fw = planes + 2 * ps;
        fps = ps;
    }

    // 2. the backward scan and the partial-sum reduction
    wkv::BwdArgs a{};
    a.w = w;
    a.u = u;
    a.k = k;
    a.v = v;
    a.gy = gy;
    a.r = r;
    a.gr = gr;
    a.gk = gk;
    a.gv = gv;
    a.gw = gw;
    a.gu = gu;
    a.fw_a = fw;
    a.fw_b = fw + fps;
    a.fw_p = fw + 2 * fps;
    a.part = planes;
    a.plane = (long)ps;
    a.ctrl = ctrl;
    a.inherit_give_up = saved == nullptr;
    a.status = reinterpret_cast<uint32_t*>(base + L.off_status);
    a.rrecs = base + L.off_rrecs;
    a.B = (int)B;
    a.T = (int)T;
    a.C = (int)C;
    a.groups_per_row = groups_per_row;
    a.n_groups = (int)n_groups;
    a.n_chunks = (int)n_chunks;
    a.n_lanes = (long)(n_groups * 64);
    int io = chunk_io(dt, C, k, v, gy);
    if (io == wkv::kIoBf16Pair && !(aligned(gk, 4) && aligned(gv, 4))) io = wkv::kIoBf16;
    if (io == wkv::kIoBf16Pair && r && !(aligned(r, 4) && aligned(gr, 4))) io = wkv::kIoBf16;
    return wkv::launch_bwd(a, io, stream) == hipSuccess ? WKV_OK : WKV_EHIP;
}

}  // namespace

extern "C" {

size_t wkv_forward_workspace_bytes(int64_t B, int64_t T, int64_t C, wkv_dtype dt, wkv_algo algo,
                                   int64_t chunk_len) {
    if (!sizes_ok(B, T, C) || !dtype_ok(dt) || !rows_ok(C, dt) || !tile_ok(chunk_len)) return (size_t)-1;
    if (algo != WKV_ALGO_AUTO && algo != WKV_ALGO_SEQ && algo != WKV_ALGO_CHUNKED) return (size_t)-1;
    if (B == 0 || T == 0 || C == 0) return 0;
    if (resolve_algo(algo, B, T, C) == WKV_ALGO_SEQ) return 0;
    return chunked_bytes_bound(B, T, C, chunk_len ? (int)chunk_len : default_tile(B, T, C));
}

wkv_status wkv_forward_workspace_init(void* ws, size_t ws_bytes, hipStream_t stream) {
    if (ws_bytes == 0) return WKV_OK;
    if (!ws || ws_bytes % 4 != 0 || !aligned(ws, 4)) return WKV_EINVAL;
    return wkv::launch_zero_words(ws, ws_bytes / 4, stream) == hipSuccess ? WKV_OK : WKV_EHIP;
}

wkv_status wkv_forward_workspace_query(const void* ws, size_t ws_bytes, uint32_t* gave_up,
                                       uint32_t* epoch, hipStream_t stream) {
    if (!ws || !gave_up || !epoch) return WKV_EINVAL;
    const uintptr_t base = align_up(reinterpret_cast<uintptr_t>(ws), kAlign);
    if (ws_bytes < (base - reinterpret_cast<uintptr_t>(ws)) + (size_t)wkv::kCtrlWords * 4)
        return WKV_EWORKSPACE;
    const uint32_t* ctrl = reinterpret_cast<const uint32_t*>(base);
    if (hipStreamSynchronize(stream) != hipSuccess) return WKV_EHIP;
    uint32_t give_up_word = 0, epoch_now = 0;
    if (hipMemcpy(&give_up_word, ctrl + wkv::kCtrlGiveUp, 4, hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(&epoch_now, ctrl + wkv::kCtrlEpoch, 4, hipMemcpyDeviceToHost) != hipSuccess)
        return WKV_EHIP;
    // a launch that gave up leaves its own epoch (one behind the counter) in the word
    const uint32_t last = (epoch_now - 1u) & wkv::kCtrlEpochMask;
    *gave_up = give_up_word == (last | wkv::kCtrlGiveUpMark) ? 1u : 0u;
    *epoch = epoch_now;
    return WKV_OK;
}

wkv_status wkv_workspace_force_give_up(void* ws, size_t ws_bytes, uint32_t launches, hipStream_t stream) {
    if (!ws) return WKV_EINVAL;
    const uintptr_t base = align_up(reinterpret_cast<uintptr_t>(ws), kAlign);
    if (ws_bytes < (base - reinterpret_cast<uintptr_t>(ws)) + (size_t)wkv::kCtrlWords * 4) return WKV_EWORKSPACE;
    uint32_t* ctrl = reinterpret_cast<uint32_t*>(base);
    return wkv::launch_set_word(ctrl + wkv::kCtrlForce, launches, stream) == hipSuccess ? WKV_OK : WKV_EHIP;
}

wkv_status wkv_forward(int64_t B, int64_t T, int64_t C, wkv_dtype dt, const float* w, const float* u,
                       const void* k, const void* v, void* y, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
    return forward_impl(B, T, C, dt, w, u, k, v, y, nullptr, nullptr, nullptr, nullptr, nullptr,
                        nullptr, ws, ws_bytes, WKV_ALGO_AUTO, 0, stream);
}

wkv_status wkv_forward_ex(int64_t B, int64_t T, int64_t C, wkv_dtype dt, const float* w,
                          const float* u, const void* k, const void* v, void* y, void* ws,
                          size_t ws_bytes, wkv_algo algo, int64_t chunk_len, hipStream_t stream) {
    return forward_impl(B, T, C, dt, w, u, k, v, y, nullptr, nullptr, nullptr, nullptr, nullptr,
                        nullptr, ws, ws_bytes, algo, chunk_len, stream);
}

wkv_status wkv_forward_state(int64_t B, int64_t T, int64_t C, wkv_dtype dt, const float* w,
                             const float* u, const void* k, const void* v, void* y,
                             const float* state_in_a, const float* state_in_b,
                             const float* state_in_p, float* state_out_a, float* state_out_b,
                             float* state_out_p, void* ws, size_t ws_bytes, wkv_algo algo,
                             int64_t chunk_len, hipStream_t stream) {
    return forward_impl(B, T, C, dt, w, u, k, v, y, state_in_a, state_in_b, state_in_p, state_out_a,
                        state_out_b, state_out_p, ws, ws_bytes, algo, chunk_len, stream);
}

size_t wkv_backward_workspace_bytes(int64_t B, int64_t T, int64_t C, wkv_dtype dt) {
    if (!sizes_ok(B, T, C) || !dtype_ok(dt) || !rows_ok(C, dt)) return (size_t)-1;
    if (B == 0 || T == 0 || C == 0) return 0;
    return backward_layout(B, T, C).total;
}

wkv_status wkv_backward(int64_t B, int64_t T, int64_t C, wkv_dtype dt, const float* w, const float* u,
                        const void* k, const void* v, const void* gy, void* gk, void* gv, float* gw,
                        float* gu, void* ws, size_t ws_bytes, hipStream_t stream) {
    return backward_impl(B, T, C, dt, w, u, k, v, gy, nullptr, 0, gk, gv, gw, gu, ws, ws_bytes, stream);
}

size_t wkv_saved_states_bytes(int64_t B, int64_t T, int64_t C) {
    if (!sizes_ok(B, T, C)) return (size_t)-1;
    if (B == 0 || T == 0 || C == 0) return 0;
    return 3 * saved_plane_bytes(B, T, C);
}

wkv_status wkv_forward_save(int64_t B, int64_t T, int64_t C, wkv_dtype dt, const float* w, const float* u,
                            const void* k, const void* v, void* y, float* saved, size_t saved_bytes, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
    if (!sizes_ok(B, T, C)) return WKV_EINVAL;
    if (!dtype_ok(dt)) return WKV_EDTYPE;
    if (!rows_ok(C, dt)) return WKV_EINVAL;
    if (B == 0 || T == 0 || C == 0) return WKV_OK;
    if (!saved || saved_bytes < 3 * saved_plane_bytes(B, T, C)) return WKV_EINVAL;
    return forward_impl(B, T, C, dt, w, u, k, v, y, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, ws,
                        ws_bytes, WKV_ALGO_CHUNKED, 0, stream, saved);
}

wkv_status wkv_backward_saved(int64_t B, int64_t T, int64_t C, wkv_dtype dt, const float* w, const float* u,
                              const void* k, const void* v, const void* gy, const float* saved,
                              size_t saved_bytes, void* gk, void* gv, float* gw, float* gu, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
    if (B > 0 && T > 0 && C > 0 && !saved) return WKV_EINVAL;
    return backward_impl(B, T, C, dt, w, u, k, v, gy, saved, saved_bytes, gk, gv, gw, gu, ws, ws_bytes, stream);
}

wkv_status wkv_forward_gated(int64_t B, int64_t T, int64_t C, wkv_dtype dt, const float* w, const float* u,
                             const void* k, const void* v, const void* r, void* z, float* saved,
                             size_t saved_bytes, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!sizes_ok(B, T, C)) return WKV_EINVAL;
    if (!dtype_ok(dt)) return WKV_EDTYPE;
    if (!rows_ok(C, dt)) return WKV_EINVAL;
    if (B == 0 || T == 0 || C == 0) return WKV_OK;
    if (!r) return WKV_EINVAL;
    if (saved && saved_bytes < 3 * saved_plane_bytes(B, T, C)) return WKV_EINVAL;
    return forward_impl(B, T, C, dt, w, u, k, v, z, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, ws,
                        ws_bytes, saved ? WKV_ALGO_CHUNKED : WKV_ALGO_AUTO, 0, stream, saved, r);
}

wkv_status wkv_backward_gated(int64_t B, int64_t T, int64_t C, wkv_dtype dt, const float* w, const float* u,
                              const void* k, const void* v, const void* r, const void* gz, const float* saved,
                              size_t saved_bytes, void* gk, void* gv, void* gr, float* gw, float* gu, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
    if (B > 0 && T > 0 && C > 0 && (!r || !gr)) {
        if (!sizes_ok(B, T, C)) return WKV_EINVAL;
        return dtype_ok(dt) ? WKV_EINVAL : WKV_EDTYPE;
    }
    return backward_impl(B, T, C, dt, w, u, k, v, gz, saved, saved_bytes, gk, gv, gw, gu, ws, ws_bytes, stream, r,
                         gr);
}

wkv_status wkv_token_shift(int64_t B, int64_t T, int64_t C, wkv_dtype dt, const void* x, const void* x_prev,
                           const float* mu, int64_t M, void* out, hipStream_t stream) {
    if (!sizes_ok(B, T, C) || M < 1 || M > wkv::kShiftMaxM) return WKV_EINVAL;
    if (!dtype_ok(dt)) return WKV_EDTYPE;
    if (B == 0 || T == 0 || C == 0) return WKV_OK;
    if (!x || !mu || !out) return WKV_EINVAL;
    if (B * T > INT_MAX || B * T * C > (int64_t)1 << 40) return WKV_EINVAL;
    const size_t vec = dt == WKV_F32 ? 4 : 8;
    const bool vector = C % (int64_t)vec == 0 && aligned(x, 16) && aligned(out, 16) && (!x_prev || aligned(x_prev, 16));
    wkv::ShiftArgs a{};
    a.x = x;
    a.x_prev = x_prev;
    a.mu = mu;
    a.out = out;
    a.B = (int)B;
    a.T = (int)T;
    a.C = (int)C;
    a.M = (int)M;
    return wkv::launch_token_shift(a, dt == WKV_F32 ? 0 : 1, vector, stream) == hipSuccess ? WKV_OK : WKV_EHIP;
}

size_t wkv_token_shift_backward_workspace_bytes(int64_t B, int64_t T, int64_t C, int64_t M) {
    if (!sizes_ok(B, T, C) || M < 1 || M > wkv::kShiftMaxM) return (size_t)-1;
    if (B == 0 || T == 0 || C == 0) return 0;
    return (size_t)wkv::token_shift_segments((long)T) * (size_t)M * (size_t)B * (size_t)C * 4 + kAlign;
}

wkv_status wkv_token_shift_backward(int64_t B, int64_t T, int64_t C, wkv_dtype dt, const void* x,
                                    const void* x_prev, const float* mu, int64_t M, const void* g, void* gx,
                                    float* gmu, void* gprev, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!sizes_ok(B, T, C) || M < 1 || M > wkv::kShiftMaxM) return WKV_EINVAL;
    if (!dtype_ok(dt)) return WKV_EDTYPE;
    if (B == 0 || C == 0) return WKV_OK;
    if (!mu || !gmu) return WKV_EINVAL;
    if (B * T > INT_MAX || B * T * C > (int64_t)1 << 40) return WKV_EINVAL;
    if (T == 0) {  // no token: dL/dmu and dL/dx_prev are zero
        if (wkv::launch_zero_words(gmu, (size_t)(M * B * C), stream) != hipSuccess) return WKV_EHIP;
        if (!gprev) return WKV_OK;
        if (dt == WKV_F32) return wkv::launch_zero_words(gprev, (size_t)(B * C), stream) == hipSuccess ? WKV_OK : WKV_EHIP;
        return wkv::launch_zero_u16(gprev, (long)(B * C), stream) == hipSuccess ? WKV_OK : WKV_EHIP;
    }
    if (!x || !g || !gx) return WKV_EINVAL;
    const size_t need = wkv_token_shift_backward_workspace_bytes(B, T, C, M);
    if (!ws || ws_bytes < need) return WKV_EWORKSPACE;
    // channels per thread: 8 (16-byte bf16 vectors, for two or more mixes), 4, or 1, as C and the
    // alignment of every [*, C] array allow
    auto fits = [&](int64_t n) {
        const size_t vb = (size_t)n * dtype_size(dt);
        return C % n == 0 && aligned(x, vb) && aligned(g, vb) && aligned(gx, vb) && (!x_prev || aligned(x_prev, vb)) &&
               (!gprev || aligned(gprev, vb));
    };
    const int vec = (dt == WKV_BF16 && M >= 2 && fits(8)) ? 8 : fits(4) ? 4 : 1;
    wkv::ShiftBwdArgs a{};
    a.x = x;
    a.x_prev = x_prev;
    a.mu = mu;
    a.g = g;
    a.gx = gx;
    a.gmu = gmu;
    a.gprev = gprev;
    a.part = reinterpret_cast<float*>(align_up(reinterpret_cast<uintptr_t>(ws), kAlign));
    a.B = (int)B;
    a.T = (int)T;
    a.C = (int)C;
    a.M = (int)M;
    return wkv::launch_token_shift_backward(a, dt == WKV_F32 ? 0 : 1, vec, stream) == hipSuccess ? WKV_OK
                                                                                                : WKV_EHIP;
}

// Linear-attention workspace: [control words][status word per chunk][records: per chunk, the
// chunk's aggregate and its inclusive state, D * M + D tagged 64-bit words each] for the one-pass
// launch, then [per chunk, D * M + D floats] for the three-launch path; a workspace serves both.
struct LaLayout {
    size_t off_status, off_recs, off_agg, total;
};

LaLayout la_layout(int64_t BH, int64_t N, int64_t D, int64_t M, wkv_dtype dt) {
    const int64_t n_chunks = ceil_div(N, wkv::la_chunk_len((int)D, (int)M, dt == WKV_F32 ? 0 : 1));
    const size_t entries = (size_t)(BH * n_chunks) * (size_t)(D * M + D);
    LaLayout L;
    L.off_status = align_up((size_t)wkv::kCtrlWords * 4, kAlign);
    L.off_recs = L.off_status + align_up((size_t)(BH * n_chunks) * 4, kAlign);
    L.off_agg = L.off_recs + align_up(entries * 2 * 8, kAlign);
    L.total = L.off_agg + entries * 4 + kAlign;  // + slack to align the base
    return L;
}

// One pass unless its chain of look-backs is the longer path.  A chunk's look-back step takes
// about 1.7 us (measured, D = M = 64, chained through a sequence), so a sequence of n chunks
// takes at least n steps; both paths are otherwise about equally bandwidth-bound, the one pass
// moving 1.2 and the three launches 1.6 times the algorithmic bytes (q, k, v read, out
// written; measured 1.63 for three launches), plus about 10 us for the two extra launches.
bool la_one_pass_auto(int64_t BH, int64_t N, int64_t D, int64_t M, wkv_dtype dt) {
    const double n_chunks = (double)ceil_div(N, wkv::la_chunk_len((int)D, (int)M, dt == WKV_F32 ? 0 : 1));
    const double bytes = (double)BH * (double)N * (double)(2 * D + 2 * M) * (dt == WKV_F32 ? 4.0 : 2.0);
    const double rate = 3.0e12;  // bytes/s either path sustains
    const double t_one = std::max(n_chunks * 1.7e-6, 1.2 * bytes / rate);
    const double t_three = 1.6 * bytes / rate + 10e-6;
    return t_one <= t_three;
}

// Feature width D and value width M of the kernels built: 32 or 64 each.
bool la_shape_ok(int64_t D, int64_t M) { return (D == 32 || D == 64) && (M == 32 || M == 64); }

size_t wkv_linear_attention_workspace_bytes(int64_t BH, int64_t N, int64_t D, int64_t M, wkv_dtype dt) {
    if (BH < 0 || N < 0 || !dtype_ok(dt)) return (size_t)-1;
    if (!la_shape_ok(D, M)) return (size_t)-1;
    if (BH == 0 || N == 0) return 0;
    return la_layout(BH, N, D, M, dt).total;
}

wkv_status wkv_linear_attention_ex(int64_t BH, int64_t N, int64_t D, int64_t M, wkv_dtype dt, const void* q,
                                   const void* k, const void* v, void* out, int feature_map, void* ws,
                                   size_t ws_bytes, wkv_la_algo algo, hipStream_t stream) {
    if (BH < 0 || N < 0 || BH > INT_MAX || N > INT_MAX) return WKV_EINVAL;
    if (!dtype_ok(dt)) return WKV_EDTYPE;
    if (!la_shape_ok(D, M)) return WKV_EINVAL;
    if (algo != WKV_LA_AUTO && algo != WKV_LA_THREE_LAUNCHES && algo != WKV_LA_ONE_PASS) return WKV_EINVAL;
    if (BH == 0 || N == 0) return WKV_OK;
    if (!q || !k || !v || !out) return WKV_EINVAL;
    // rows are moved with 16-byte accesses
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return WKV_EINVAL;
    const int64_t n_chunks = ceil_div(N, wkv::la_chunk_len((int)D, (int)M, dt == WKV_F32 ? 0 : 1));
    if (BH * n_chunks > INT_MAX || BH * N * std::max(D, M) > ((int64_t)1 << 40)) return WKV_EINVAL;
    const size_t need = wkv_linear_attention_workspace_bytes(BH, N, D, M, dt);
    if (!ws || ws_bytes < need) return WKV_EWORKSPACE;
    wkv::LaArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    const LaLayout L = la_layout(BH, N, D, M, dt);
    char* base = reinterpret_cast<char*>(align_up(reinterpret_cast<uintptr_t>(ws), kAlign));
    a.ctrl = reinterpret_cast<uint32_t*>(base);
    a.status = reinterpret_cast<uint32_t*>(base + L.off_status);
    a.recs = base + L.off_recs;
    a.agg = reinterpret_cast<float*>(base + L.off_agg);
    a.BH = (int)BH;
    a.N = (int)N;
    a.D = (int)D;
    a.M = (int)M;
    a.n_chunks = (int)n_chunks;
    a.feature = feature_map ? 1 : 0;
    a.one_pass = algo == WKV_LA_ONE_PASS || (algo == WKV_LA_AUTO && la_one_pass_auto(BH, N, D, M, dt));
    return wkv::launch_linear_attention(a, dt == WKV_F32 ? 0 : 1, stream) == hipSuccess ? WKV_OK : WKV_EHIP;
}

wkv_status wkv_linear_attention(int64_t BH, int64_t N, int64_t D, int64_t M, wkv_dtype dt, const void* q,
                                const void* k, const void* v, void* out, int feature_map, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
    return wkv_linear_attention_ex(BH, N, D, M, dt, q, k, v, out, feature_map, ws, ws_bytes, WKV_LA_AUTO, stream);
}

wkv_status wkv_step(int64_t N, int64_t G, int64_t C, wkv_dtype dt, const float* w, const float* u,
                    const void* k, const void* v, float* a, float* b, float* p, void* y,
                    hipStream_t stream) {
    if (N < 0 || G < 0 || C < 0) return WKV_EINVAL;
    if (!dtype_ok(dt)) return WKV_EDTYPE;
    if (N == 0 || G == 0 || C == 0) return WKV_OK;
    if (G > INT_MAX || C > INT_MAX || G * C > INT_MAX) return WKV_EINVAL;
    if (N > (int64_t)(LONG_MAX / 4) / (G * C)) return WKV_EINVAL;
    if (!w || !u || !k || !v || !a || !b || !p || !y) return WKV_EINVAL;
    const size_t elt = dtype_size(dt);
    int nch = 1;
    if (C % 4 == 0 && aligned(w, 16) && aligned(u, 16) && aligned(a, 16) && aligned(b, 16) &&
        aligned(p, 16) && aligned(k, 4 * elt) && aligned(v, 4 * elt) && aligned(y, 4 * elt))
        nch = 4;
    wkv::StepArgs s{};
    s.w = w;
    s.u = u;
    s.k = k;
    s.v = v;
    s.a = a;
    s.b = b;
    s.p = p;
    s.y = y;
    s.n_lanes = (long)(N * G * C);
    s.GC = (int)(G * C);
    return wkv::launch_step(s, dt == WKV_F32 ? 0 : 1, nch, stream) == hipSuccess ? WKV_OK : WKV_EHIP;
}

const char* wkv_status_string(wkv_status s) {
    switch (s) {
        case WKV_OK: return "WKV_OK";
        case WKV_EINVAL: return "WKV_EINVAL: invalid size, pointer, algorithm or chunk length";
        case WKV_EDTYPE: return "WKV_EDTYPE: unknown dtype";
        case WKV_EWORKSPACE: return "WKV_EWORKSPACE: workspace missing or too small";
        case WKV_EHIP: return "WKV_EHIP: a HIP launch failed";
    }
    return "unknown wkv_status";
}

}  // extern "C"
