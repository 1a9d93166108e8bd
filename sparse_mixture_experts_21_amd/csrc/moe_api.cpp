// C ABI of libmoe.so: argument validation, capacity, workspace layout and the
// launch sequence of every stage.  All validation happens before the first
// HIP call, so a rejected call enqueues nothing (and needs no GPU).
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "moe_internal.h"

namespace moe {

static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

int device_cus() {
    static std::atomic<int> cus[64];
    int d = 0;
    if (hipGetDevice(&d) != hipSuccess || d < 0 || d >= 64) return 256;
    int n = cus[d].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, d) != hipSuccess ||
            n <= 0)
            n = 256;
        cus[d].store(n, std::memory_order_relaxed);
    }
    return n;
}

WsLayout ws_layout(const moe_problem_t& p) {
    WsLayout L;
    std::memset(&L, 0, sizeof L);
    const size_t T = (size_t)p.T, H = (size_t)p.H, E = (size_t)p.E, k = (size_t)p.k,
                 F = (size_t)p.F;
    const size_t s = p.dtype == MOE_DTYPE_BF16 ? 2 : 4;
    L.nblk_route = (p.T + kRouteTok - 1) / kRouteTok;
    L.nchunk = (p.T + kChunkTok - 1) / kChunkTok;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off += align256(bytes);
        return o;
    };
    const size_t nb = (size_t)L.nblk_route, nc = (size_t)L.nchunk;
    L.blk_psum = take(nb * E * 4);
    L.blk_lse2 = take(nb * 4);
    L.blk_cnt = take(nb * E * 4);
    L.fin_sum = take((E + 1) * 8);
    L.fin_cnt = take(E * 8);
    L.small_disp = take(route_small_fits(p) ? (E + 1 + 2 * T * k) * 4 : 0);
    L.route_bytes = off;
    L.chunk_hist = take(nc * E * 4);
    L.chunk_base = take(nc * E * 4);
    L.col_tot = take(E * 4);
    L.gemm_part = take(gemm_partial_bytes(p));
    L.permute_bytes = off;
    L.ffn_bytes = 0;
    L.logits = 0;                 // moe_forward never stores logits in the workspace
    L.topk_idx = take(T * k * 4);
    L.topk_w = take(T * k * 4);
    L.counts = take(E * 4);
    L.offsets = take((E + 1) * 4);
    L.pos = take(T * k * 4);
    L.row_token = take(T * k * 4);
    L.xp = 0;                     // moe_forward gathers x inside the first GEMM
    L.h = take(T * k * F * s);
    L.y = take(T * k * H * s);
    L.total = off;
    return L;
}

}  // namespace moe

using namespace moe;

namespace {

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }
bool opt_ok(const void* ptr) { return ptr == nullptr || aligned16(ptr); }

moe_status_t check_problem(const moe_problem_t* p) {
    if (!p) return MOE_ERR_INVALID_ARG;
    if (p->T < 1 || p->H < 1 || p->F < 1 || p->E < 1 || p->k < 1 || p->k > p->E)
        return MOE_ERR_INVALID_ARG;
    if (p->dtype != MOE_DTYPE_F32 && p->dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID_ARG;
    if (p->activation != MOE_ACT_GELU && p->activation != MOE_ACT_SILU) return MOE_ERR_INVALID_ARG;
    if (std::isnan(p->capacity_factor)) return MOE_ERR_INVALID_ARG;
    if (p->E > kMaxE || p->k > kMaxK) return MOE_ERR_UNSUPPORTED;
    if (p->T > (int64_t)0x7fffffff / p->k) return MOE_ERR_UNSUPPORTED;
    const int vec = p->dtype == MOE_DTYPE_BF16 ? 8 : 4;
    if (p->H % vec != 0 || p->F % vec != 0) return MOE_ERR_UNSUPPORTED;
    if (p->dtype == MOE_DTYPE_BF16) {
        // 32-bit buffer-resource ranges (offsets at or past 2^31 mean "out of
        // range"): the token rows the first GEMM gathers from, one expert's
        // weight block, the gate, and the GEMM's tile grid.
        const int64_t lim = (int64_t)1 << 31;
        if (p->T * p->H * 2 >= lim) return MOE_ERR_UNSUPPORTED;
        if ((int64_t)p->H * p->F * 2 >= lim) return MOE_ERR_UNSUPPORTED;
        if ((int64_t)p->E * p->H * 2 >= lim) return MOE_ERR_UNSUPPORTED;
        const int64_t tiles = (p->T * p->k / 64 + p->E + 1) * (((int64_t)std::max(p->H, p->F) + 255) / 256);
        if (tiles + 256 >= lim) return MOE_ERR_UNSUPPORTED;   // + a round of K slices
    }
    return MOE_OK;
}

// ---------------------------------------------------------------- expert choice
constexpr int64_t kEcMaxGroup = 32768;    // keys of one (expert, group) held in LDS

int64_t ec_capacity_of(const moe_problem_t& p, int64_t group) {
    const double cf = p.capacity_factor > 0.0 ? p.capacity_factor : 1.0;
    double c = std::ceil(cf * (double)group * (double)p.k / (double)p.E);
    if (c < 1.0) c = 1.0;
    if (c > (double)group) c = (double)group;
    return (int64_t)c;
}

// Workspace of the expert-choice calls: the router's regions of ws_layout
// first, then logits, probs, rowof, sel, offsets, the router's top-k scratch,
// the GEMM partials and the h / y rows.  `pg` is the problem the grouped GEMMs
// see: k rounded up so that T * k covers the A selected rows, no capacity.
struct EcLayout {
    size_t logits, probs, rowof, sel, offsets, topk_idx, topk_w, part, h, y;
    size_t route_total, total;
    int64_t C, A;
    moe_problem_t pg;
    WsLayout L;
};

EcLayout ec_layout(const moe_problem_t& p, int64_t group) {
    EcLayout X;
    X.L = ws_layout(p);
    const size_t T = (size_t)p.T, E = (size_t)p.E, k = (size_t)p.k, H = (size_t)p.H,
                 F = (size_t)p.F;
    const size_t s = p.dtype == MOE_DTYPE_BF16 ? 2 : 4;
    X.C = ec_capacity_of(p, group);
    X.A = (int64_t)E * (p.T / group) * X.C;
    X.pg = p;
    X.pg.k = (int32_t)((X.A + p.T - 1) / p.T);
    X.pg.capacity_factor = 0.0;
    size_t off = X.L.route_bytes;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off += align256(bytes);
        return o;
    };
    const size_t A = (size_t)X.A;
    X.logits = take(T * E * 4);
    X.probs = take(T * E * 4);
    X.rowof = take(T * E * 4);
    X.sel = take(A * 4);
    X.offsets = take((E + 1) * 4);
    X.topk_idx = take(T * k * 4);
    X.topk_w = take(T * k * 4);
    X.route_total = off;
    X.part = take(gemm_partial_bytes(X.pg));
    X.h = take(A * F * s);
    X.y = take(A * H * s);
    X.total = off;
    return X;
}

moe_status_t check_group(const moe_problem_t* p, int64_t group) {
    moe_status_t st = check_problem(p);
    if (st != MOE_OK) return st;
    if (group < 1 || p->T % group != 0) return MOE_ERR_INVALID_ARG;
    if (group > kEcMaxGroup) return MOE_ERR_UNSUPPORTED;
    const int64_t lim = (int64_t)1 << 31;
    if (p->T * (int64_t)p->E >= lim) return MOE_ERR_UNSUPPORTED;
    const int64_t A = (int64_t)p->E * (p->T / group) * ec_capacity_of(*p, group);
    const int64_t tiles = (A / 64 + p->E + 1) * (((int64_t)std::max(p->H, p->F) + 255) / 256);
    if (A >= lim || tiles + 256 >= lim) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

int64_t capacity_of(const moe_problem_t& p) {
    if (!(p.capacity_factor > 0.0)) return p.T;
    const double c = std::ceil(p.capacity_factor * (double)(p.T * (int64_t)p.k) / (double)p.E);
    if (c >= 9.0e18) return INT64_MAX;
    return (int64_t)c;
}

// ---------------------------------------------------------------- training
// Workspace of moe_forward_train / moe_backward: the forward's layout (whose
// routing, dispatch, h and y the backward reads) followed by the fp32
// logits, the rows ga = act'(a) at the first GEMM's pre-activation a, and the
// backward's scratch: dy, dl, da,
// dxe (the expert part of dx per kept row), the gathered rows xp and the
// partial sums of the gate gradients.
struct TrainLayout {
    WsLayout L;
    size_t logits, ga, dy, dl, da, dxe, xp, gpart, gpb, total;
};

TrainLayout train_layout(const moe_problem_t& p) {
    TrainLayout X;
    X.L = ws_layout(p);
    const size_t T = (size_t)p.T, H = (size_t)p.H, E = (size_t)p.E, k = (size_t)p.k,
                 F = (size_t)p.F;
    const size_t nc = (size_t)bwd_gate_chunks(p);
    size_t off = X.L.total;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off += align256(bytes);
        return o;
    };
    X.logits = take(T * E * 4);
    X.ga = take(T * k * F * 2);
    X.dy = take(T * k * H * 2);
    X.dl = take(T * E * 4);
    X.da = take(T * k * F * 2);
    X.dxe = take(T * k * H * 2);
    X.xp = take(T * k * H * 2);
    X.gpart = take(nc * H * E * 4);
    X.gpb = take(nc * E * 4);
    X.total = off;
    return X;
}

// The backward runs on bf16 storage; its weight-gradient GEMMs address one
// expert's rows of h, dy, xp and da through 32-bit buffer offsets.
moe_status_t check_train(const moe_problem_t* p) {
    moe_status_t st = check_problem(p);
    if (st != MOE_OK) return st;
    if (p->dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED;
    if (p->T * p->k * (int64_t)std::max(p->H, p->F) * 2 >= ((int64_t)1 << 31))
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

// The forward's launch sequence; NULL outputs live in the workspace.  hgrad
// (nullable): also keep act' at the first GEMM's pre-activation rows.
moe_status_t forward_impl(const moe_problem_t& P, const WsLayout& L, char* w, const void* x,
                          const void* Wg, const void* bg, const void* W1, const void* b1,
                          const void* W2, const void* b2, void* out, float* losses,
                          float* logits, int32_t* topk_idx, float* topk_w, int32_t* counts,
                          int32_t* offsets, int32_t* pos, void* hgrad, hipStream_t stream,
                          hipEvent_t* stage_events) {
    const moe_problem_t* p = &P;
    int32_t* idx = topk_idx ? topk_idx : reinterpret_cast<int32_t*>(w + L.topk_idx);
    float* tw = topk_w ? topk_w : reinterpret_cast<float*>(w + L.topk_w);
    int32_t* cnt = counts ? counts : reinterpret_cast<int32_t*>(w + L.counts);
    int32_t* off = offsets ? offsets : reinterpret_cast<int32_t*>(w + L.offsets);
    int32_t* ps = pos ? pos : reinterpret_cast<int32_t*>(w + L.pos);
    int32_t* rt = reinterpret_cast<int32_t*>(w + L.row_token);
    void* h = w + L.h;
    void* y = w + L.y;

    auto ev = [&](int i) -> hipError_t {
        return stage_events && stage_events[i] ? hipEventRecord(stage_events[i], stream)
                                              : hipSuccess;
    };
    hipError_t e = ev(MOE_EV_ROUTE);
    if (route_small_fits(*p)) {
        // a few tokens: routing and dispatch in one launch (the permute stage is empty)
        if (e == hipSuccess)
            e = launch_route_small(*p, capacity_of(*p), x, Wg, bg, logits, idx, tw, cnt, losses,
                                   off, ps, rt, stream);
        if (e == hipSuccess) e = ev(MOE_EV_PERMUTE);
    } else {
        if (e == hipSuccess)
            e = launch_route(*p, L, w, x, Wg, bg, logits, false, idx, tw, cnt, losses, false,
                             stream);
        if (e == hipSuccess) e = ev(MOE_EV_PERMUTE);
        if (e == hipSuccess)
            e = launch_permute(*p, L, w, capacity_of(*p), x, idx, off, ps, rt, nullptr, cnt,
                               losses, stream);
    }
    if (e == hipSuccess) e = ev(MOE_EV_FFN_UP);
    float* part = reinterpret_cast<float*>(w + L.gemm_part);
    hipEvent_t up_fix = stage_events ? stage_events[MOE_EV_FFN_UP_FIXUP] : nullptr;
    hipEvent_t down_fix = stage_events ? stage_events[MOE_EV_FFN_DOWN_FIXUP] : nullptr;
    if (e == hipSuccess) e = launch_ffn_up(*p, x, rt, off, W1, b1, h, hgrad, part, up_fix, stream);
    // Inference (bf16): the combine finishes the second GEMM's cut tiles from
    // their K-slice partials, so that GEMM needs no fixup launch.  Training
    // keeps y whole for the backward.
    const bool cut_in_combine = hgrad == nullptr && p->dtype == MOE_DTYPE_BF16;
    if (e == hipSuccess) e = ev(MOE_EV_FFN_DOWN);
    if (e == hipSuccess)
        e = launch_ffn_down(*p, h, off, W2, b2, y, part, down_fix, stream, !cut_in_combine);
    if (e == hipSuccess) e = ev(MOE_EV_COMBINE);
    if (e == hipSuccess)
        e = cut_in_combine ? launch_combine_cut(*p, y, ps, tw, idx, off, b2, part, out, stream)
                           : launch_combine(*p, y, ps, tw, out, stream);
    if (e == hipSuccess) e = ev(MOE_EV_END);
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// ---------------------------------------------------------------- fixed scratch
// The workspace of moe_forward_noalloc: a file-scope device array that every
// GPU the library runs on holds until the process ends.  In host code
// `scratch` names a host-side stand-in, never the device memory: its device
// address is looked up once per device (with that device current) and only
// that address is handed to kernels.
static __device__ __align__(256) char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of `scratch` on the device that owns `stream`.
hipError_t scratch_address(hipStream_t stream, char** out) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    int dev = cur;
    if (stream) {
        hipDevice_t sd = 0;
        e = hipStreamGetDevice(stream, &sd);
        if (e != hipSuccess) return e;
        dev = (int)sd;
    }
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t r = hipSetDevice(cur);
            if (e == hipSuccess) e = r;
        }
        if (e != hipSuccess) return e;
        if (!ptr) return hipErrorInvalidSymbol;
        g_scratch_dev[dev] = ptr;
    }
    *out = static_cast<char*>(g_scratch_dev[dev]);
    return hipSuccess;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status_t s) {
    // a C caller may pass any int: read the raw value (in C++ a value outside
    // the enumerators would be undefined behaviour)
    static_assert(sizeof(moe_status_t) == sizeof(int), "status is int-sized");
    int v = 0;
    std::memcpy(&v, &s, sizeof v);
    switch (v) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported problem (outside the kernel envelope)";
        case MOE_ERR_WORKSPACE: return "workspace too small";
        case MOE_ERR_HIP: return "HIP launch or event failure";
    }
    return "unknown status";
}

moe_status_t moe_capacity(const moe_problem_t* p, int64_t* cap) {
    moe_status_t st = check_problem(p);
    if (st != MOE_OK) return st;
    if (!cap) return MOE_ERR_INVALID_ARG;
    *cap = capacity_of(*p);
    return MOE_OK;
}

moe_status_t moe_workspace_bytes(const moe_problem_t* p, size_t* bytes) {
    moe_status_t st = check_problem(p);
    if (st != MOE_OK) return st;
    if (!bytes) return MOE_ERR_INVALID_ARG;
    *bytes = ws_layout(*p).total;
    return MOE_OK;
}

moe_status_t moe_route(const moe_problem_t* p, const void* x, const void* Wg, const void* bg,
                       float* logits, int32_t* topk_idx, float* topk_w, int32_t* counts,
                       float* losses, uint32_t flags, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
    moe_status_t st = check_problem(p);
    if (st != MOE_OK) return st;
    if (flags & ~MOE_ROUTE_LOGITS_IN) return MOE_ERR_INVALID_ARG;
    const bool logits_in = (flags & MOE_ROUTE_LOGITS_IN) != 0;
    if (!topk_idx || !topk_w || !counts || !losses || !ws) return MOE_ERR_INVALID_ARG;
    if (logits_in ? !logits : (!x || !Wg)) return MOE_ERR_INVALID_ARG;
    if (!opt_ok(x) || !opt_ok(Wg) || !opt_ok(bg) || !opt_ok(logits) || !aligned16(topk_idx) ||
        !aligned16(topk_w) || !aligned16(counts) || !aligned16(losses) || !aligned16(ws))
        return MOE_ERR_UNSUPPORTED;
    const WsLayout L = ws_layout(*p);
    if (ws_bytes < L.route_bytes) return MOE_ERR_WORKSPACE;
    hipError_t e;
    if (!logits_in && route_small_fits(*p)) {
        // the launch moe_forward takes for a few tokens, so that the stages
        // reproduce its routing bit for bit; its dispatch outputs are dropped
        int32_t* sd = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + L.small_disp);
        const int64_t pairs = p->T * p->k;
        e = launch_route_small(*p, capacity_of(*p), x, Wg, bg, logits, topk_idx, topk_w, counts,
                               losses, sd, sd + p->E + 1, sd + p->E + 1 + pairs, stream);
    } else {
        e = launch_route(*p, L, static_cast<char*>(ws), x, Wg, bg, logits, logits_in, topk_idx,
                         topk_w, counts, losses, true, stream);
    }
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status_t moe_permute(const moe_problem_t* p, const void* x, const int32_t* topk_idx,
                         int32_t* offsets, int32_t* pos, int32_t* row_token, void* xp, void* ws,
                         size_t ws_bytes, hipStream_t stream) {
    moe_status_t st = check_problem(p);
    if (st != MOE_OK) return st;
    if (!x || !topk_idx || !offsets || !pos || !row_token || !xp || !ws)
        return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(topk_idx) || !aligned16(offsets) || !aligned16(pos) ||
        !aligned16(row_token) || !aligned16(xp) || !aligned16(ws))
        return MOE_ERR_UNSUPPORTED;
    const WsLayout L = ws_layout(*p);
    if (ws_bytes < L.permute_bytes) return MOE_ERR_WORKSPACE;
    hipError_t e = launch_permute(*p, L, static_cast<char*>(ws), capacity_of(*p), x, topk_idx,
                                  offsets, pos, row_token, xp, nullptr, nullptr, stream);
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status_t moe_expert_ffn(const moe_problem_t* p, const void* xp, const int32_t* offsets,
                            const void* W1, const void* b1, const void* W2, const void* b2,
                            void* h, void* y, void* ws, size_t ws_bytes, hipStream_t stream) {
    moe_status_t st = check_problem(p);
    if (st != MOE_OK) return st;
    if (!xp || !offsets || !W1 || !W2 || !h || !y) return MOE_ERR_INVALID_ARG;
    if (!aligned16(xp) || !aligned16(offsets) || !aligned16(W1) || !opt_ok(b1) ||
        !aligned16(W2) || !opt_ok(b2) || !aligned16(h) || !aligned16(y))
        return MOE_ERR_UNSUPPORTED;
    // the workspace is optional here: with it, the ragged last round of tiles
    // is cut along K (see moe_workspace_bytes)
    float* part = (ws && aligned16(ws) && ws_bytes >= gemm_partial_bytes(*p))
                      ? static_cast<float*>(ws) : nullptr;
    hipError_t e = launch_ffn_up(*p, xp, nullptr, offsets, W1, b1, h, nullptr, part, nullptr, stream);
    if (e == hipSuccess) e = launch_ffn_down(*p, h, offsets, W2, b2, y, part, nullptr, stream);
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status_t moe_combine(const moe_problem_t* p, const void* y, const int32_t* pos,
                         const float* topk_w, void* out, hipStream_t stream) {
    moe_status_t st = check_problem(p);
    if (st != MOE_OK) return st;
    if (!y || !pos || !topk_w || !out) return MOE_ERR_INVALID_ARG;
    if (!aligned16(y) || !aligned16(pos) || !aligned16(topk_w) || !aligned16(out))
        return MOE_ERR_UNSUPPORTED;
    hipError_t e = launch_combine(*p, y, pos, topk_w, out, stream);
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status_t moe_forward(const moe_problem_t* p, const void* x, const void* Wg, const void* bg,
                         const void* W1, const void* b1, const void* W2, const void* b2,
                         void* out, float* losses, float* logits, int32_t* topk_idx,
                         float* topk_w, int32_t* counts, int32_t* offsets, int32_t* pos,
                         void* ws, size_t ws_bytes, hipStream_t stream,
                         hipEvent_t* stage_events) {
    moe_status_t st = check_problem(p);
    if (st != MOE_OK) return st;
    if (!x || !Wg || !W1 || !W2 || !out || !losses || !ws) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(Wg) || !opt_ok(bg) || !aligned16(W1) || !opt_ok(b1) ||
        !aligned16(W2) || !opt_ok(b2) || !aligned16(out) || !aligned16(losses) ||
        !opt_ok(logits) || !opt_ok(topk_idx) || !opt_ok(topk_w) || !opt_ok(counts) ||
        !opt_ok(offsets) || !opt_ok(pos) || !aligned16(ws))
        return MOE_ERR_UNSUPPORTED;
    const WsLayout L = ws_layout(*p);
    if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    return forward_impl(*p, L, static_cast<char*>(ws), x, Wg, bg, W1, b1, W2, b2, out, losses,
                        logits, topk_idx, topk_w, counts, offsets, pos, nullptr, stream,
                        stage_events);
}

moe_status_t moe_forward_noalloc(const moe_problem_t* p, const void* x, const void* Wg,
                                 const void* bg, const void* W1, const void* b1, const void* W2,
                                 const void* b2, void* out, float* losses, float* logits,
                                 int32_t* topk_idx, float* topk_w, int32_t* counts,
                                 int32_t* offsets, int32_t* pos, hipStream_t stream,
                                 hipEvent_t* stage_events) {
    moe_status_t st = check_problem(p);
    if (st != MOE_OK) return st;
    if (!x || !Wg || !W1 || !W2 || !out || !losses) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(Wg) || !opt_ok(bg) || !aligned16(W1) || !opt_ok(b1) ||
        !aligned16(W2) || !opt_ok(b2) || !aligned16(out) || !aligned16(losses) ||
        !opt_ok(logits) || !opt_ok(topk_idx) || !opt_ok(topk_w) || !opt_ok(counts) ||
        !opt_ok(offsets) || !opt_ok(pos))
        return MOE_ERR_UNSUPPORTED;
    const WsLayout L = ws_layout(*p);
    if (L.total > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
    char* w = nullptr;
    if (scratch_address(stream, &w) != hipSuccess) return MOE_ERR_HIP;
    // every region of the workspace is written before it is read within one
    // forward, so the previous call's contents need no clearing
    return forward_impl(*p, L, w, x, Wg, bg, W1, b1, W2, b2, out, losses, logits, topk_idx,
                        topk_w, counts, offsets, pos, nullptr, stream, stage_events);
}

moe_status_t moe_ec_capacity(const moe_problem_t* p, int64_t group, int64_t* C) {
    moe_status_t st = check_group(p, group);
    if (st != MOE_OK) return st;
    if (!C) return MOE_ERR_INVALID_ARG;
    *C = ec_capacity_of(*p, group);
    return MOE_OK;
}

moe_status_t moe_ec_workspace_bytes(const moe_problem_t* p, int64_t group, size_t* bytes) {
    moe_status_t st = check_group(p, group);
    if (st != MOE_OK) return st;
    if (!bytes) return MOE_ERR_INVALID_ARG;
    *bytes = ec_layout(*p, group).total;
    return MOE_OK;
}

moe_status_t moe_route_expert_choice(const moe_problem_t* p, int64_t group, const void* x,
                                     const void* Wg, const void* bg, float* logits,
                                     uint32_t flags, float* probs, int32_t* sel, int32_t* rowof,
                                     int32_t* offsets, void* ws, size_t ws_bytes,
                                     hipStream_t stream) {
    moe_status_t st = check_group(p, group);
    if (st != MOE_OK) return st;
    if (flags & ~MOE_ROUTE_LOGITS_IN) return MOE_ERR_INVALID_ARG;
    const bool logits_in = (flags & MOE_ROUTE_LOGITS_IN) != 0;
    if (!probs || !sel || !rowof || !offsets || !ws) return MOE_ERR_INVALID_ARG;
    if (logits_in ? !logits : (!x || !Wg)) return MOE_ERR_INVALID_ARG;
    if (!opt_ok(x) || !opt_ok(Wg) || !opt_ok(bg) || !opt_ok(logits) || !aligned16(probs) ||
        !aligned16(sel) || !aligned16(rowof) || !aligned16(offsets) || !aligned16(ws))
        return MOE_ERR_UNSUPPORTED;
    const EcLayout X = ec_layout(*p, group);
    if (ws_bytes < X.route_total) return MOE_ERR_WORKSPACE;
    char* w = static_cast<char*>(ws);
    float* lg = logits ? logits : reinterpret_cast<float*>(w + X.logits);
    hipError_t e = hipSuccess;
    if (!logits_in)
        e = launch_route(*p, X.L, w, x, Wg, bg, lg, false,
                         reinterpret_cast<int32_t*>(w + X.topk_idx),
                         reinterpret_cast<float*>(w + X.topk_w), nullptr, nullptr, false, stream);
    if (e == hipSuccess)
        e = launch_expert_choice(*p, group, X.C, lg, probs, sel, rowof, offsets, stream);
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status_t moe_forward_expert_choice(const moe_problem_t* p, int64_t group, const void* x,
                                       const void* Wg, const void* bg, const void* W1,
                                       const void* b1, const void* W2, const void* b2,
                                       void* out, float* logits, float* probs, int32_t* sel,
                                       int32_t* rowof, void* ws, size_t ws_bytes,
                                       hipStream_t stream, hipEvent_t* stage_events) {
    moe_status_t st = check_group(p, group);
    if (st != MOE_OK) return st;
    if (!x || !Wg || !W1 || !W2 || !out || !ws) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(Wg) || !opt_ok(bg) || !aligned16(W1) || !opt_ok(b1) ||
        !aligned16(W2) || !opt_ok(b2) || !aligned16(out) || !opt_ok(logits) || !opt_ok(probs) ||
        !opt_ok(sel) || !opt_ok(rowof) || !aligned16(ws))
        return MOE_ERR_UNSUPPORTED;
    const EcLayout X = ec_layout(*p, group);
    if (ws_bytes < X.total) return MOE_ERR_WORKSPACE;
    char* w = static_cast<char*>(ws);
    float* lg = logits ? logits : reinterpret_cast<float*>(w + X.logits);
    float* pr = probs ? probs : reinterpret_cast<float*>(w + X.probs);
    int32_t* sl = sel ? sel : reinterpret_cast<int32_t*>(w + X.sel);
    int32_t* ro = rowof ? rowof : reinterpret_cast<int32_t*>(w + X.rowof);
    int32_t* off = reinterpret_cast<int32_t*>(w + X.offsets);
    float* part = reinterpret_cast<float*>(w + X.part);
    void* h = w + X.h;
    void* y = w + X.y;
    moe_problem_t pc = *p;                 // combine: one slot per expert
    pc.k = p->E;

    auto ev = [&](int i) -> hipError_t {
        return stage_events && stage_events[i] ? hipEventRecord(stage_events[i], stream)
                                              : hipSuccess;
    };
    hipEvent_t up_fix = stage_events ? stage_events[MOE_EV_FFN_UP_FIXUP] : nullptr;
    hipEvent_t down_fix = stage_events ? stage_events[MOE_EV_FFN_DOWN_FIXUP] : nullptr;
    hipError_t e = ev(MOE_EV_ROUTE);
    if (e == hipSuccess)
        e = launch_route(*p, X.L, w, x, Wg, bg, lg, false,
                         reinterpret_cast<int32_t*>(w + X.topk_idx),
                         reinterpret_cast<float*>(w + X.topk_w), nullptr, nullptr, false, stream);
    if (e == hipSuccess) e = ev(MOE_EV_PERMUTE);
    if (e == hipSuccess) e = launch_expert_choice(*p, group, X.C, lg, pr, sl, ro, off, stream);
    if (e == hipSuccess) e = ev(MOE_EV_FFN_UP);
    if (e == hipSuccess) e = launch_ffn_up(X.pg, x, sl, off, W1, b1, h, nullptr, part, up_fix, stream);
    if (e == hipSuccess) e = ev(MOE_EV_FFN_DOWN);
    if (e == hipSuccess) e = launch_ffn_down(X.pg, h, off, W2, b2, y, part, down_fix, stream);
    if (e == hipSuccess) e = ev(MOE_EV_COMBINE);
    if (e == hipSuccess) e = launch_combine(pc, y, ro, pr, out, stream);
    if (e == hipSuccess) e = ev(MOE_EV_END);
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status_t moe_train_workspace_bytes(const moe_problem_t* p, size_t* bytes) {
    moe_status_t st = check_train(p);
    if (st != MOE_OK) return st;
    if (!bytes) return MOE_ERR_INVALID_ARG;
    *bytes = train_layout(*p).total;
    return MOE_OK;
}

moe_status_t moe_forward_train(const moe_problem_t* p, const void* x, const void* Wg,
                               const void* bg, const void* W1, const void* b1, const void* W2,
                               const void* b2, void* out, float* losses, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
    moe_status_t st = check_train(p);
    if (st != MOE_OK) return st;
    if (!x || !Wg || !W1 || !W2 || !out || !losses || !ws) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(Wg) || !opt_ok(bg) || !aligned16(W1) || !opt_ok(b1) ||
        !aligned16(W2) || !opt_ok(b2) || !aligned16(out) || !aligned16(losses) || !aligned16(ws))
        return MOE_ERR_UNSUPPORTED;
    const TrainLayout X = train_layout(*p);
    if (ws_bytes < X.total) return MOE_ERR_WORKSPACE;
    char* w = static_cast<char*>(ws);
    return forward_impl(*p, X.L, w, x, Wg, bg, W1, b1, W2, b2, out, losses,
                        reinterpret_cast<float*>(w + X.logits), nullptr, nullptr, nullptr,
                        nullptr, nullptr, w + X.ga, stream, nullptr);
}

moe_status_t moe_backward(const moe_problem_t* p, const void* x, const void* Wg, const void* W1,
                          const void* W2, const void* dout, float g_aux, float g_z, void* dx,
                          float* dWg, float* dbg, float* dW1, float* db1, float* dW2, float* db2,
                          void* ws, size_t ws_bytes, hipStream_t stream,
                          hipEvent_t* stage_events) {
    moe_status_t st = check_train(p);
    if (st != MOE_OK) return st;
    if (!x || !Wg || !W1 || !W2 || !dout || !dx || !dWg || !dW1 || !dW2 || !ws)
        return MOE_ERR_INVALID_ARG;
    if (std::isnan(g_aux) || std::isnan(g_z)) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(Wg) || !aligned16(W1) || !aligned16(W2) || !aligned16(dout) ||
        !aligned16(dx) || !aligned16(dWg) || !opt_ok(dbg) || !aligned16(dW1) || !opt_ok(db1) ||
        !aligned16(dW2) || !opt_ok(db2) || !aligned16(ws))
        return MOE_ERR_UNSUPPORTED;
    const TrainLayout X = train_layout(*p);
    if (ws_bytes < X.total) return MOE_ERR_WORKSPACE;
    char* w = static_cast<char*>(ws);
    const WsLayout& L = X.L;
    auto* idx = reinterpret_cast<const int32_t*>(w + L.topk_idx);
    auto* tw = reinterpret_cast<const float*>(w + L.topk_w);
    auto* cnt = reinterpret_cast<const int32_t*>(w + L.counts);
    auto* off = reinterpret_cast<const int32_t*>(w + L.offsets);
    auto* ps = reinterpret_cast<const int32_t*>(w + L.pos);
    auto* lg = reinterpret_cast<const float*>(w + X.logits);
    float* dl = reinterpret_cast<float*>(w + X.dl);
    void* dy = w + X.dy;
    void* da = w + X.da;
    void* dxe = w + X.dxe;
    void* xp = w + X.xp;
    const int H = p->H, F = p->F;

    auto ev = [&](int i) -> hipError_t {
        return stage_events && stage_events[i] ? hipEventRecord(stage_events[i], stream)
                                              : hipSuccess;
    };
    // dw, dy rows and the router's dl; then the two data-gradient GEMMs and dx
    hipError_t e = ev(MOE_BEV_TOKEN);
    if (e == hipSuccess)
        e = launch_bwd_token(*p, dout, w + L.y, ps, idx, tw, lg, cnt, g_aux, g_z, dy, dl, stream);
    if (e == hipSuccess) e = ev(MOE_BEV_DGRAD_DA);
    if (e == hipSuccess) e = launch_bwd_dgrad(*p, true, dy, off, W2, w + X.ga, da, H, F, stream);
    if (e == hipSuccess) e = ev(MOE_BEV_DGRAD_DXE);
    if (e == hipSuccess) e = launch_bwd_dgrad(*p, false, da, off, W1, nullptr, dxe, F, H, stream);
    if (e == hipSuccess) e = ev(MOE_BEV_DX);
    if (e == hipSuccess) e = launch_bwd_dx(*p, dxe, ps, dl, Wg, dx, stream);
    // weight gradients
    if (e == hipSuccess) e = ev(MOE_BEV_GATHER);
    if (e == hipSuccess) e = launch_gather(*p, x, ps, xp, stream);
    if (e == hipSuccess) e = ev(MOE_BEV_WGRAD_W2);
    if (e == hipSuccess) e = launch_bwd_wgrad(*p, w + L.h, dy, off, F, H, dW2, stream);
    if (e == hipSuccess) e = ev(MOE_BEV_WGRAD_W1);
    if (e == hipSuccess) e = launch_bwd_wgrad(*p, xp, da, off, H, F, dW1, stream);
    if (e == hipSuccess) e = ev(MOE_BEV_BIAS);
    if (e == hipSuccess && db2) e = launch_bwd_colsum(*p, dy, off, H, db2, stream);
    if (e == hipSuccess && db1) e = launch_bwd_colsum(*p, da, off, F, db1, stream);
    if (e == hipSuccess) e = ev(MOE_BEV_GATE);
    if (e == hipSuccess)
        e = launch_bwd_gate(*p, x, dl, reinterpret_cast<float*>(w + X.gpart),
                            reinterpret_cast<float*>(w + X.gpb), dWg, dbg, stream);
    if (e == hipSuccess) e = ev(MOE_BEV_END);
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // extern "C"
