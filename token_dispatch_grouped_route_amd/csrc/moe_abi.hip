// C ABI of the gfx950 MoE expert-layer library: argument checks, workspace layout and stage
// launches on the caller's stream.  Declarations and the meaning of every argument are in
// include/moe.h.  No entry point allocates, frees, copies to or from the host, or waits.
#include <string.h>

#include <mutex>

#include "moe_internal.h"

using namespace moe;

namespace {

constexpr size_t kWsAlign = 256;
constexpr int kMxSlotK = 256;   // K advances 256 per slot in the MX GEMMs (and the FP4 scale layout groups four 64-deep steps)

size_t align_up(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int32_t check_shape(const moe_shape* s) {
    if (!s) return MOE_ERR_NULL;
    if (s->block_m != 32 && s->block_m != 64 && s->block_m != 128 && s->block_m != 256) return MOE_ERR_BLOCK_M;
    if (s->T < 0 || s->H <= 0 || s->I <= 0 || s->E <= 0 || s->EL < 1 || s->EL > 1024 || s->e_lo < 0 ||
        s->k < 1 || s->k > 32)
        return MOE_ERR_SHAPE;
    if (static_cast<int64_t>(s->e_lo) + s->EL > s->E) return MOE_ERR_SHAPE;
    if (s->H % 128 != 0 || s->I % 128 != 0) return MOE_ERR_SHAPE;
    // row and element indices stay far inside int32 / int64 ranges
    const int64_t rows = static_cast<int64_t>(s->T) * s->k + static_cast<int64_t>(s->EL) * s->block_m;
    if (rows > (int64_t(1) << 28) || s->H > (1 << 20) || s->I > (1 << 20)) return MOE_ERR_SHAPE;
    // byte offsets inside one expert's packed weights are 32-bit in the GEMM tile loaders
    if (4 * static_cast<int64_t>(s->I) * s->H >= (int64_t(1) << 31)) return MOE_ERR_SHAPE;
    return MOE_OK;
}

int32_t layout_of(const moe_shape* s, moe_ws_layout* L) {
    const int32_t st = check_shape(s);
    if (st != MOE_OK) return st;
    memset(L, 0, sizeof(*L));
    const int64_t BM = s->block_m;
    const int64_t pairs = static_cast<int64_t>(s->T) * s->k;
    const int64_t R = (pairs + static_cast<int64_t>(s->EL) * (BM - 1) + BM - 1) / BM * BM;
    const int64_t rc = route_chunk_for(pairs, s->EL);
    const int64_t chunks = pairs > 0 ? (pairs + rc - 1) / rc : 1;
    const size_t H = s->H, I = s->I, EL = s->EL;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align_up(off + bytes);
        return o;
    };
    L->rows_capacity = R;
    L->num_blocks = R / BM;
    L->counts = take(4 * EL);
    L->padded_offsets = take(4 * (EL + 1));
    L->row_pair = take(4 * static_cast<size_t>(R));
    L->pair_row = take(4 * static_cast<size_t>(pairs));
    L->tile_expert = take(4 * static_cast<size_t>(R / BM));
    L->tok_nloc = take(4 * static_cast<size_t>(s->T));
    L->meta = take(16);
    L->act = take(2 * static_cast<size_t>(R) * I);
    L->stage = take(4 * static_cast<size_t>(R) * H);
    if (s->train) {
        L->hgu = take(4 * static_cast<size_t>(R) * 2 * I);
        L->dact = take(4 * static_cast<size_t>(R) * I);
        L->dhgu = take(2 * static_cast<size_t>(R) * 2 * I);
        L->dhgu_lo = take(2 * static_cast<size_t>(R) * 2 * I);
        L->wact = take(2 * static_cast<size_t>(R) * I);
        L->wact_lo = take(2 * static_cast<size_t>(R) * I);
    }
    L->zeros = take(2 * (H > 2 * I ? H : 2 * I));
    L->tile_sync = take(4 * static_cast<size_t>(kMaxGrid));
    L->scratch = take(4 * static_cast<size_t>(chunks) * (EL + 1));
    if (s->train) L->dtw_part = take(4 * static_cast<size_t>(R) * (I / 128));
    L->total_bytes = off;
    return MOE_OK;
}

bool is_gfx950() {
    static int cached[64] = {0};   // 0 unknown, 1 yes, 2 no
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
    if (!cached[dev]) {
        hipDeviceProp_t prop;
        bool ok = hipGetDeviceProperties(&prop, dev) == hipSuccess &&
                  strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        cached[dev] = ok ? 1 : 2;
    }
    return cached[dev] == 1;
}

// Shared preamble of every device entry point: shape, workspace size/alignment, device.
int32_t prepare(const moe_shape* s, const void* ws, size_t ws_bytes, bool need_train, Dims* d, Ws* w,
                moe_ws_layout* L) {
    const int32_t st = layout_of(s, L);
    if (st != MOE_OK) return st;
    if (!ws) return MOE_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(ws) & (kWsAlign - 1)) != 0) return MOE_ERR_ALIGN;
    if (ws_bytes < L->total_bytes) return MOE_ERR_WORKSPACE;
    if (need_train && !s->train) return MOE_ERR_WORKSPACE;
    if (!is_gfx950()) return MOE_ERR_DEVICE;
    *d = Dims{s->T, s->H, s->I, s->E, s->e_lo, s->EL, s->k, s->block_m};
    char* b = static_cast<char*>(const_cast<void*>(ws));
    w->counts = reinterpret_cast<int32_t*>(b + L->counts);
    w->offsets = reinterpret_cast<int32_t*>(b + L->padded_offsets);
    w->row_pair = reinterpret_cast<int32_t*>(b + L->row_pair);
    w->pair_row = reinterpret_cast<int32_t*>(b + L->pair_row);
    w->tile_expert = reinterpret_cast<int32_t*>(b + L->tile_expert);
    w->tok_nloc = reinterpret_cast<int32_t*>(b + L->tok_nloc);
    w->meta = reinterpret_cast<int32_t*>(b + L->meta);
    w->act = reinterpret_cast<uint16_t*>(b + L->act);
    w->stage = reinterpret_cast<float*>(b + L->stage);
    w->hgu = s->train ? reinterpret_cast<float*>(b + L->hgu) : nullptr;
    w->dact = s->train ? reinterpret_cast<float*>(b + L->dact) : nullptr;
    w->dhgu = s->train ? reinterpret_cast<uint16_t*>(b + L->dhgu) : nullptr;
    w->dhgu_lo = s->train ? reinterpret_cast<uint16_t*>(b + L->dhgu_lo) : nullptr;
    w->wact = s->train ? reinterpret_cast<uint16_t*>(b + L->wact) : nullptr;
    w->wact_lo = s->train ? reinterpret_cast<uint16_t*>(b + L->wact_lo) : nullptr;
    w->dtw_part = s->train ? reinterpret_cast<float*>(b + L->dtw_part) : nullptr;
    w->dtw_cols = s->I / 128;
    const int64_t pairs = static_cast<int64_t>(s->T) * s->k;
    w->route_chunk = route_chunk_for(pairs, s->EL);
    w->num_chunks = static_cast<int32_t>(pairs > 0 ? (pairs + w->route_chunk - 1) / w->route_chunk : 1);
    w->chunk_hist = reinterpret_cast<int32_t*>(b + L->scratch);
    w->chunk_dropped = w->chunk_hist + static_cast<int64_t>(w->num_chunks) * s->EL;
    w->zeros = reinterpret_cast<uint16_t*>(b + L->zeros);
    w->tile_sync = reinterpret_cast<int32_t*>(b + L->tile_sync);
    w->zero_len = s->H > 2 * s->I ? s->H : 2 * s->I;
    w->rows_cap = L->rows_capacity;
    w->num_blocks = static_cast<int32_t>(L->num_blocks);
    return MOE_OK;
}

int32_t launched(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH; }

}  // namespace

extern "C" {

const char* moe_status_string(int32_t status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_NULL: return "a required pointer is NULL";
        case MOE_ERR_SHAPE: return "a size is out of the supported range";
        case MOE_ERR_BLOCK_M: return "block_m must be 32, 64, 128 or 256";
        case MOE_ERR_WORKSPACE: return "workspace too small or without the train buffers";
        case MOE_ERR_ALIGN: return "misaligned pointer (16 bytes; workspace 256 bytes)";
        case MOE_ERR_LAUNCH: return "kernel launch failed";
        case MOE_ERR_DEVICE: return "current device is not gfx950 or HIP failed";
        case MOE_ERR_SCRATCH: return "the shape needs more workspace than the fixed scratch of moe_forward_noalloc";
        default: return "unknown status";
    }
}

size_t moe_workspace_bytes(const moe_shape* shape) {
    moe_ws_layout L;
    return layout_of(shape, &L) == MOE_OK ? L.total_bytes : 0;
}

int32_t moe_workspace_layout(const moe_shape* shape, moe_ws_layout* out) {
    if (!out) return MOE_ERR_NULL;
    return layout_of(shape, out);
}

int32_t moe_preferred_block_m(const moe_shape* s) {
    if (!s || s->E <= 0 || s->T < 0 || s->k < 1) return 64;
    // mean rows per expert under uniform routing; a block at most half that keeps the expected
    // padding of each segment (half a block) under about a quarter of its rows
    const double mean = static_cast<double>(s->T) * s->k / s->E;
    if (mean >= 512) return 256;
    if (mean >= 256) return 128;
    return 64;
}

int32_t moe_pack_weights(const moe_shape* shape, const uint16_t* w1, const uint16_t* w2, uint16_t* w1p,
                         uint16_t* w2p, void* stream) {
    const int32_t st = check_shape(shape);
    if (st != MOE_OK) return st;
    if ((w1 == nullptr) != (w1p == nullptr) || (w2 == nullptr) != (w2p == nullptr)) return MOE_ERR_NULL;
    if ((w1 && w1 == w1p) || (w2 && w2 == w2p)) return MOE_ERR_SHAPE;   // not in place
    if (!aligned16(w1) || !aligned16(w2) || !aligned16(w1p) || !aligned16(w2p)) return MOE_ERR_ALIGN;
    if (!is_gfx950()) return MOE_ERR_DEVICE;
    const Dims d{shape->T, shape->H, shape->I, shape->E, shape->e_lo, shape->EL, shape->k, shape->block_m};
    return launched(launch_pack(d, w1, w2, w1p, w2p, static_cast<hipStream_t>(stream)));
}

int32_t moe_unpack_weights(const moe_shape* shape, const uint16_t* w1p, const uint16_t* w2p, uint16_t* w1,
                           uint16_t* w2, void* stream) {
    const int32_t st = check_shape(shape);
    if (st != MOE_OK) return st;
    if ((w1 == nullptr) != (w1p == nullptr) || (w2 == nullptr) != (w2p == nullptr)) return MOE_ERR_NULL;
    if ((w1 && w1 == w1p) || (w2 && w2 == w2p)) return MOE_ERR_SHAPE;   // not in place
    if (!aligned16(w1) || !aligned16(w2) || !aligned16(w1p) || !aligned16(w2p)) return MOE_ERR_ALIGN;
    if (!is_gfx950()) return MOE_ERR_DEVICE;
    const Dims d{shape->T, shape->H, shape->I, shape->E, shape->e_lo, shape->EL, shape->k, shape->block_m};
    return launched(launch_unpack(d, w1p, w2p, w1, w2, static_cast<hipStream_t>(stream)));
}

int32_t moe_route_prologue(const moe_shape* shape, const int32_t* topk_idx, void* ws, size_t ws_bytes,
                           void* stream) {
    Dims d;
    Ws w;
    moe_ws_layout L;
    int32_t st = prepare(shape, ws, ws_bytes, false, &d, &w, &L);
    if (st != MOE_OK) return st;
    if (!topk_idx && shape->T > 0) return MOE_ERR_NULL;
    if (!aligned4(topk_idx)) return MOE_ERR_ALIGN;
    return launched(launch_route(d, topk_idx, w, static_cast<hipStream_t>(stream)));
}

int32_t moe_dispatch_gemm1(const moe_shape* shape, const uint16_t* x, const uint16_t* w1p, void* ws,
                           size_t ws_bytes, uint16_t* act_out, float* hgu_out, void* stream) {
    Dims d;
    Ws w;
    moe_ws_layout L;
    int32_t st = prepare(shape, ws, ws_bytes, false, &d, &w, &L);
    if (st != MOE_OK) return st;
    if ((!x && shape->T > 0) || !w1p || (!act_out && !hgu_out)) return MOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(w1p) || !aligned16(act_out) || !aligned16(hgu_out)) return MOE_ERR_ALIGN;
    return launched(launch_gemm1(d, x, w1p, w, act_out, hgu_out, static_cast<hipStream_t>(stream)));
}

int32_t moe_swiglu(const moe_shape* shape, const float* hgu, const void* ws, size_t ws_bytes, uint16_t* act,
                   void* stream) {
    Dims d;
    Ws w;
    moe_ws_layout L;
    int32_t st = prepare(shape, ws, ws_bytes, false, &d, &w, &L);
    if (st != MOE_OK) return st;
    if (!hgu || !act) return MOE_ERR_NULL;
    if (!aligned16(hgu) || !aligned16(act)) return MOE_ERR_ALIGN;
    return launched(launch_swiglu(d, hgu, w, act, static_cast<hipStream_t>(stream)));
}

int32_t moe_gemm2_combine(const moe_shape* shape, const uint16_t* act, const uint16_t* w2p, const float* topk_w,
                          void* ws, size_t ws_bytes, uint16_t* y, void* stream) {
    Dims d;
    Ws w;
    moe_ws_layout L;
    int32_t st = prepare(shape, ws, ws_bytes, false, &d, &w, &L);
    if (st != MOE_OK) return st;
    if (!act || !w2p || ((!topk_w || !y) && shape->T > 0)) return MOE_ERR_NULL;
    if (!aligned16(act) || !aligned16(w2p) || !aligned4(topk_w) || !aligned16(y)) return MOE_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = launch_gemm2_combine(d, act, w2p, topk_w, w, y, s);
    if (e == hipSuccess) e = launch_combine_finish(d, w, y, s);
    return launched(e);
}

int32_t moe_forward(const moe_shape* shape, const uint16_t* x, const int32_t* topk_idx, const float* topk_w,
                    const uint16_t* w1p, const uint16_t* w2p, void* ws, size_t ws_bytes, uint16_t* y,
                    void* stream) {
    Dims d;
    Ws w;
    moe_ws_layout L;
    int32_t st = prepare(shape, ws, ws_bytes, false, &d, &w, &L);
    if (st != MOE_OK) return st;
    if (!w1p || !w2p || ((!x || !topk_idx || !topk_w || !y) && shape->T > 0)) return MOE_ERR_NULL;
    if (!aligned16(x) || !aligned4(topk_idx) || !aligned4(topk_w) || !aligned16(w1p) || !aligned16(w2p) ||
        !aligned16(y))
        return MOE_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = launch_route(d, topk_idx, w, s);
    if (e == hipSuccess) e = launch_gemm1(d, x, w1p, w, w.act, w.hgu, s);
    if (e == hipSuccess) e = launch_gemm2_combine(d, w.act, w2p, topk_w, w, y, s);
    if (e == hipSuccess) e = launch_combine_finish(d, w, y, s);
    return launched(e);
}

// ---------------------------------------------------------------------------------------------
// Allocation-free forward: the workspace is a fixed device array of this file
// ---------------------------------------------------------------------------------------------
// The array itself.  In host code its name is only a stand-in for the device symbol: the device
// address of each GPU's copy comes from hipGetSymbolAddress, once per device, and only that
// address is passed to kernels.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on the first call per device).
int32_t scratch_of_current_device(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_DEVICE;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}
}  // namespace

int32_t moe_forward_noalloc(const moe_shape* shape, const uint16_t* x, const int32_t* topk_idx, const float* topk_w,
                            const uint16_t* w1p, const uint16_t* w2p, uint16_t* y, void* stream) {
    moe_ws_layout L;
    int32_t st = layout_of(shape, &L);
    if (st != MOE_OK) return st;
    if (shape->train) return MOE_ERR_SHAPE;
    if (L.total_bytes > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
    if (!w1p || !w2p || ((!x || !topk_idx || !topk_w || !y) && shape->T > 0)) return MOE_ERR_NULL;
    if (!aligned16(x) || !aligned4(topk_idx) || !aligned4(topk_w) || !aligned16(w1p) || !aligned16(w2p) ||
        !aligned16(y))
        return MOE_ERR_ALIGN;
    if (!is_gfx950()) return MOE_ERR_DEVICE;
    void* ws = nullptr;
    st = scratch_of_current_device(&ws);
    if (st != MOE_OK) return st;
    Dims d;
    Ws w;
    st = prepare(shape, ws, MOE_NOALLOC_SCRATCH_BYTES, false, &d, &w, &L);
    if (st != MOE_OK) return st;
    // the same stages as moe_forward; the prologue rewrites every table, the tile counters and the
    // zero row, and the GEMMs write every row they later read, so stale contents of the array
    // from an earlier call do not matter
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = launch_route(d, topk_idx, w, s);
    if (e == hipSuccess) e = launch_gemm1(d, x, w1p, w, w.act, nullptr, s);
    if (e == hipSuccess) e = launch_gemm2_combine(d, w.act, w2p, topk_w, w, y, s);
    if (e == hipSuccess) e = launch_combine_finish(d, w, y, s);
    return launched(e);
}

int32_t moe_bwd_gemm2_dgrad(const moe_shape* shape, const uint16_t* dy, const float* topk_w, const uint16_t* w2p,
                            void* ws, size_t ws_bytes, int32_t fuse_swiglu_bwd, float* dtopk_w, void* stream) {
    Dims d;
    Ws w;
    moe_ws_layout L;
    int32_t st = prepare(shape, ws, ws_bytes, true, &d, &w, &L);
    if (st != MOE_OK) return st;
    if (!w2p || ((!dy || !topk_w) && shape->T > 0)) return MOE_ERR_NULL;
    if (!aligned16(dy) || !aligned4(topk_w) || !aligned16(w2p) || !aligned4(dtopk_w)) return MOE_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = launch_dgrad(d, dy, topk_w, w2p, w, fuse_swiglu_bwd != 0, dtopk_w != nullptr, s);
    if (e == hipSuccess && dtopk_w) e = launch_dtopk_w_finish(d, w, dtopk_w, s);
    return launched(e);
}

int32_t moe_bwd_gemm1_dgrad_combine(const moe_shape* shape, const uint16_t* w1p, void* ws, size_t ws_bytes,
                                    uint16_t* dx, void* stream) {
    Dims d;
    Ws w;
    moe_ws_layout L;
    int32_t st = prepare(shape, ws, ws_bytes, true, &d, &w, &L);
    if (st != MOE_OK) return st;
    if (!w1p || (!dx && shape->T > 0)) return MOE_ERR_NULL;
    if (!aligned16(w1p) || !aligned16(dx)) return MOE_ERR_ALIGN;
    return launched(launch_dgrad1(d, w1p, w, dx, static_cast<hipStream_t>(stream)));
}

int32_t moe_swiglu_bwd(const moe_shape* shape, void* ws, size_t ws_bytes, void* stream) {
    Dims d;
    Ws w;
    moe_ws_layout L;
    int32_t st = prepare(shape, ws, ws_bytes, true, &d, &w, &L);
    if (st != MOE_OK) return st;
    return launched(launch_swiglu_bwd(d, w, static_cast<hipStream_t>(stream)));
}

int32_t moe_wgrad2(const moe_shape* shape, const uint16_t* dy, void* ws, size_t ws_bytes, uint16_t* dw2p,
                   void* stream) {
    Dims d;
    Ws w;
    moe_ws_layout L;
    int32_t st = prepare(shape, ws, ws_bytes, true, &d, &w, &L);
    if (st != MOE_OK) return st;
    if (!dw2p || (!dy && shape->T > 0)) return MOE_ERR_NULL;
    if (!aligned16(dy) || !aligned16(dw2p)) return MOE_ERR_ALIGN;
    return launched(launch_wgrad2(d, dy, w, dw2p, static_cast<hipStream_t>(stream)));
}

int32_t moe_wgrad1(const moe_shape* shape, const uint16_t* x, void* ws, size_t ws_bytes, uint16_t* dw1p,
                   void* stream) {
    Dims d;
    Ws w;
    moe_ws_layout L;
    int32_t st = prepare(shape, ws, ws_bytes, true, &d, &w, &L);
    if (st != MOE_OK) return st;
    if (!dw1p || (!x && shape->T > 0)) return MOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(dw1p)) return MOE_ERR_ALIGN;
    return launched(launch_wgrad1(d, x, w, dw1p, static_cast<hipStream_t>(stream)));
}

int32_t moe_backward(const moe_shape* shape, const uint16_t* x, const uint16_t* dy, const float* topk_w,
                     const uint16_t* w1p, const uint16_t* w2p, void* ws, size_t ws_bytes, uint16_t* dw1p,
                     uint16_t* dw2p, uint16_t* dx, float* dtopk_w, void* stream) {
    Dims d;
    Ws w;
    moe_ws_layout L;
    int32_t st = prepare(shape, ws, ws_bytes, true, &d, &w, &L);
    if (st != MOE_OK) return st;
    if (!w2p || !dw1p || !dw2p || ((!x || !dy || !topk_w) && shape->T > 0)) return MOE_ERR_NULL;
    if (dx && !w1p) return MOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(dy) || !aligned4(topk_w) || !aligned16(w1p) || !aligned16(w2p) ||
        !aligned16(dw1p) || !aligned16(dw2p) || !aligned16(dx) || !aligned4(dtopk_w))
        return MOE_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = launch_dgrad(d, dy, topk_w, w2p, w, 1, dtopk_w != nullptr, s);
    if (e == hipSuccess && dtopk_w) e = launch_dtopk_w_finish(d, w, dtopk_w, s);
    if (e == hipSuccess) e = launch_wgrad2(d, dy, w, dw2p, s);
    if (e == hipSuccess) e = launch_wgrad1(d, x, w, dw1p, s);
    if (e == hipSuccess && dx) e = launch_dgrad1(d, w1p, w, dx, s);
    return launched(e);
}

int32_t moe_mx_cast_fp8(int64_t rows, int32_t cols, const uint16_t* x, uint8_t* codes, uint8_t* scales,
                        void* stream) {
    if (rows < 0 || cols <= 0 || cols % 32 != 0) return MOE_ERR_SHAPE;
    if (rows > 0 && (!x || !codes || !scales)) return MOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(codes)) return MOE_ERR_ALIGN;
    if (!is_gfx950()) return MOE_ERR_DEVICE;
    return launched(launch_mx_cast_fp8(rows, cols, x, codes, scales, static_cast<hipStream_t>(stream)));
}

static bool mx_shape_ok(const moe_shape* shape) {
    return shape->H % kMxSlotK == 0 && shape->I % kMxSlotK == 0;
}

int32_t moe_mx_pack_weights(const moe_shape* shape, const uint16_t* w1, const uint16_t* w2, uint8_t* w1q,
                            uint8_t* w1s, uint8_t* w2q, uint8_t* w2s, void* stream) {
    const int32_t st = check_shape(shape);
    if (st != MOE_OK) return st;
    if (!mx_shape_ok(shape)) return MOE_ERR_SHAPE;
    if ((w1 == nullptr) != (w1q == nullptr) || (w1 == nullptr) != (w1s == nullptr) ||
        (w2 == nullptr) != (w2q == nullptr) || (w2 == nullptr) != (w2s == nullptr))
        return MOE_ERR_NULL;
    if (!aligned16(w1) || !aligned16(w2) || !aligned16(w1q) || !aligned16(w2q)) return MOE_ERR_ALIGN;
    if (!is_gfx950()) return MOE_ERR_DEVICE;
    const Dims d{shape->T, shape->H, shape->I, shape->E, shape->e_lo, shape->EL, shape->k, shape->block_m};
    return launched(launch_mx_pack(d, w1, w2, w1q, w1s, w2q, w2s, static_cast<hipStream_t>(stream)));
}

int32_t moe_mx_dispatch_gemm1(const moe_shape* shape, const uint8_t* xq, const uint8_t* xs, const uint8_t* w1q,
                              const uint8_t* w1s, float clamp, void* ws, size_t ws_bytes, void* stream) {
    Dims d;
    Ws w;
    moe_ws_layout L;
    int32_t st = prepare(shape, ws, ws_bytes, false, &d, &w, &L);
    if (st != MOE_OK) return st;
    if (!mx_shape_ok(shape)) return MOE_ERR_SHAPE;
    if (!w1q || !w1s || ((!xq || !xs) && shape->T > 0)) return MOE_ERR_NULL;
    if (!aligned16(xq) || !aligned4(xs) || !aligned16(w1q)) return MOE_ERR_ALIGN;
    return launched(launch_mx_gemm1(d, xq, xs, w1q, w1s, w, clamp, static_cast<hipStream_t>(stream)));
}

int32_t moe_mx_gemm2_combine(const moe_shape* shape, const uint8_t* w2q, const uint8_t* w2s, const float* topk_w,
                             void* ws, size_t ws_bytes, uint16_t* y, void* stream) {
    Dims d;
    Ws w;
    moe_ws_layout L;
    int32_t st = prepare(shape, ws, ws_bytes, false, &d, &w, &L);
    if (st != MOE_OK) return st;
    if (!mx_shape_ok(shape)) return MOE_ERR_SHAPE;
    if (!w2q || !w2s || ((!topk_w || !y) && shape->T > 0)) return MOE_ERR_NULL;
    if (!aligned16(w2q) || !aligned4(topk_w) || !aligned16(y)) return MOE_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = launch_mx_gemm2(d, w2q, w2s, topk_w, w, y, s);
    if (e == hipSuccess) e = launch_combine_finish(d, w, y, s);
    return launched(e);
}

int32_t moe_forward_mx(const moe_shape* shape, const uint8_t* xq, const uint8_t* xs, const int32_t* topk_idx,
                       const float* topk_w, const uint8_t* w1q, const uint8_t* w1s, const uint8_t* w2q,
                       const uint8_t* w2s, float clamp, void* ws, size_t ws_bytes, uint16_t* y, void* stream) {
    Dims d;
    Ws w;
    moe_ws_layout L;
    int32_t st = prepare(shape, ws, ws_bytes, false, &d, &w, &L);
    if (st != MOE_OK) return st;
    if (!mx_shape_ok(shape)) return MOE_ERR_SHAPE;
    if (!w1q || !w1s || !w2q || !w2s || ((!xq || !xs || !topk_idx || !topk_w || !y) && shape->T > 0)) return MOE_ERR_NULL;
    if (!aligned16(xq) || !aligned4(xs) || !aligned4(topk_idx) || !aligned4(topk_w) || !aligned16(w1q) ||
        !aligned16(w2q) || !aligned16(y))
        return MOE_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = launch_route(d, topk_idx, w, s);
    if (e == hipSuccess) e = launch_mx_gemm1(d, xq, xs, w1q, w1s, w, clamp, s);
    if (e == hipSuccess) e = launch_mx_gemm2(d, w2q, w2s, topk_w, w, y, s);
    if (e == hipSuccess) e = launch_combine_finish(d, w, y, s);
    return launched(e);
}

}  // extern "C"
