// C-ABI entry points: argument checks, workspace carve-up and launch sequencing.
// Every call only queues kernels on the caller's stream; nothing here
// allocates, frees or synchronises.
#include <climits>
#include <map>
#include <memory>
#include <mutex>
#include <utility>

#include "common.h"

using namespace moe_kernels;

namespace {

constexpr size_t ALIGN = 256;
inline size_t align_up(size_t v) { return (v + ALIGN - 1) & ~(ALIGN - 1); }

moe_status check_shape(const moe_shape* s, moe_dims* out) {
    if (!s) return MOE_ERR_INVALID_ARGUMENT;
    if (s->T < 0 || s->d < 1 || s->m < 1 || s->E < 1 || s->k < 1 || s->k > s->E) return MOE_ERR_INVALID_ARGUMENT;
    if (s->capacity < 0 || s->m_shared < 0) return MOE_ERR_INVALID_ARGUMENT;
    if (s->gate_mode != MOE_GATE_RENORM && s->gate_mode != MOE_GATE_SWITCH) return MOE_ERR_INVALID_ARGUMENT;
    if (s->dtype != MOE_F32 && s->dtype != MOE_BF16) return MOE_ERR_INVALID_ARGUMENT;
    if (s->E > 1024 || s->k > 32) return MOE_ERR_UNSUPPORTED;
    if (s->T * (int64_t)s->k > (int64_t)INT_MAX) return MOE_ERR_UNSUPPORTED;
    if (s->dtype == MOE_BF16 && (s->d % 8 || s->m % 8 || s->m_shared % 8)) return MOE_ERR_UNSUPPORTED;
    if ((s->accept_by_gate != 0 && s->accept_by_gate != 1) || (s->renorm_survivors != 0 && s->renorm_survivors != 1) ||
        (s->reroute != 0 && s->reroute != 1))
        return MOE_ERR_INVALID_ARGUMENT;
    if (s->reroute && s->accept_by_gate) return MOE_ERR_UNSUPPORTED;   // rerouting is read with token order
    if (out) {
        out->T = s->T;
        out->d = s->d;
        out->m = s->m;
        out->E = s->E;
        out->k = s->k;
        out->C = s->capacity > 0 ? s->capacity : (int)(s->T > 0 ? s->T : 1);
        out->gate_mode = s->gate_mode;
        out->dtype = s->dtype;
        out->m_shared = s->m_shared;
        out->accept_by_gate = s->accept_by_gate;
        out->renorm_survivors = s->renorm_survivors;
        out->reroute = s->reroute;
    }
    return MOE_OK;
}

int64_t max_rows(const moe_dims& d) {
    const int64_t a = d.T * d.k, b = (int64_t)d.E * d.C;
    return a < b ? a : b;
}

size_t elem(const moe_dims& d) { return d.dtype == MOE_BF16 ? 2 : 4; }

// At most one row per token and expert, and at most C per expert.
int64_t group_rows(const moe_dims& d) { return d.T < d.C ? d.T : d.C; }

// Bytes of the K-split partials of H beyond the first (S - 1 blocks of R d fp32)
// when GEMM2 splits K for this shape; of GEMM1's gate / up partials.
size_t partial_bytes(const moe_dims& d) {
    const int64_t R = max_rows(d);
    const int S = gemm2_splits(d.dtype, R, d.E, d.d, d.m, group_rows(d));
    return S > 1 ? align_up(sizeof(float) * (S - 1) * R * d.d) : 0;
}
size_t g1_part_bytes(const moe_dims& d) {
    return align_up(gemm1_part_bytes(d.dtype, max_rows(d), d.E, d.m, d.d, group_rows(d)));
}
// [tile prefix | h | GEMM1 partials | H partials]
size_t ffn_ws(const moe_dims& d) {
    return align_up(gemm_ws_bytes(d.E)) + align_up((size_t)max_rows(d) * d.m * elem(d)) + g1_part_bytes(d) +
           partial_bytes(d);
}
// moe_expert_gemm1 alone: [tile prefix | GEMM1 partials]
size_t gemm1_ws(const moe_dims& d) { return align_up(gemm_ws_bytes(d.E)) + g1_part_bytes(d); }
// moe_expert_gemm2 alone: [tile prefix | H partials]
size_t gemm2_ws(const moe_dims& d) { return align_up(gemm_ws_bytes(d.E)) + partial_bytes(d); }
// moe_route's workspace: the sync words, then the router's own part
size_t route_ws(const moe_dims& d) { return MOE_SYNC_BYTES + align_up(route_ws_bytes(d)); }
// moe_route's workspace, then the [T, E] fp32 probabilities
size_t route_stats_ws(const moe_dims& d) { return route_ws(d) + align_up((size_t)d.T * d.E * sizeof(float)); }
// shared expert: [tile prefix | h | GEMM1 partials | s partials] (one group of T rows)
size_t shared_g1_bytes(const moe_dims& d) {
    return align_up(gemm1_part_bytes(d.dtype, d.T, 1, d.m_shared, d.d, d.T));
}
size_t shared_g2_bytes(const moe_dims& d) {
    const int S = gemm2_splits(d.dtype, d.T, 1, d.d, d.m_shared, d.T);
    return S > 1 ? align_up(sizeof(float) * (S - 1) * d.T * d.d) : 0;
}
size_t shared_ws(const moe_dims& d) {
    return align_up(gemm_ws_bytes(1)) + align_up((size_t)d.T * d.m_shared * elem(d)) + shared_g1_bytes(d) +
           shared_g2_bytes(d);
}

struct ForwardWs {
    int32_t* sync;
    int32_t* offsets;
    int32_t* row_of;
    int32_t* src_token;
    void* x_perm;
    float* H;
    float* s;
    void* route;
    void* dispatch;
    void* ffn;
    void* shared;
    size_t total;
};

bool gather_rows(const moe_dims& d) { return gemm1_gather_ok(d.dtype, d.m, d.d, d.T); }

ForwardWs carve_forward(const moe_dims& d, void* base) {
    ForwardWs w{};
    char* p = static_cast<char*>(base);
    size_t off = 0;
    auto take = [&](size_t bytes) -> void* {
        void* r = p ? p + off : nullptr;
        off += align_up(bytes);
        return r;
    };
    const int64_t R = max_rows(d);
    // GEMM1 reads the grouped rows in place through src_token where it can (then
    // src_token is padded by one row tile and there is no x_perm)
    const bool gather = gather_rows(d);
    w.sync = static_cast<int32_t*>(take(MOE_SYNC_BYTES));   // fixed place: the same for every shape
    w.offsets = static_cast<int32_t*>(take(sizeof(int32_t) * (d.E + 1)));
    w.row_of = static_cast<int32_t*>(take(sizeof(int32_t) * d.T * moe_paths(d)));
    w.src_token = static_cast<int32_t*>(take(sizeof(int32_t) * (R + (gather ? 256 : 0))));
    w.x_perm = gather ? nullptr : take((size_t)R * d.d * elem(d));
    w.H = static_cast<float*>(take(sizeof(float) * R * d.d));
    w.s = d.m_shared ? static_cast<float*>(take(sizeof(float) * d.T * d.d)) : nullptr;
    w.route = take(route_ws_bytes(d));
    w.dispatch = take(dispatch_ws_bytes(d));
    w.ffn = take(ffn_ws(d));
    w.shared = d.m_shared ? take(shared_ws(d)) : nullptr;
    w.total = off;
    return w;
}

inline moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// The shared expert depends on x alone, so moe_forward runs it on a second stream
// concurrently with the routed path: an event on the caller's stream forks it,
// another joins it before the combine.  Each caller stream gets a side stream of
// its own (default priority, non-blocking, on the caller stream's device) and
// its own two events, created on first use and kept for the process (they hold
// no device memory), so calls on different caller streams share no state: one
// stream's graph capture never reaches another stream's eager calls.  The
// entry's mutex keeps one call's record / wait sequence together when several
// host threads launch on the same caller stream.
struct SideStream {
    hipStream_t stream = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
    std::mutex mu;
};
constexpr int MAX_DEVICES = 64;
std::mutex g_side_mu;   // guards the map only
std::map<std::pair<int, hipStream_t>, std::unique_ptr<SideStream>> g_side;

// The side stream paired with caller stream `st` (its device made current only
// while the stream and events are created).
hipError_t side_stream(hipStream_t st, SideStream** out) {
    hipDevice_t dev = 0;
    hipError_t e = hipStreamGetDevice(st, &dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(g_side_mu);
    std::unique_ptr<SideStream>& slot = g_side[{(int)dev, st}];
    if (!slot) {
        std::unique_ptr<SideStream> s(new SideStream);
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        e = hipEventCreateWithFlags(&s->fork, hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&s->join, hipEventDisableTiming);
        if (e == hipSuccess) e = hipStreamCreateWithFlags(&s->stream, hipStreamNonBlocking);
        const hipError_t r = cur != dev ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess || r != hipSuccess) {   // leave no half-made entry behind
            if (s->fork) (void)hipEventDestroy(s->fork);
            if (s->join) (void)hipEventDestroy(s->join);
            if (s->stream) (void)hipStreamDestroy(s->stream);
            g_side.erase({(int)dev, st});
            return e != hipSuccess ? e : r;
        }
        slot = std::move(s);
    }
    *out = slot.get();
    return hipSuccess;
}

#define MOE_CHECK_HIP(expr)                        \
    do {                                           \
        hipError_t e_ = (expr);                    \
        if (e_ != hipSuccess) return MOE_ERR_HIP;  \
    } while (0)

// K-split partials of H still to be added (np blocks of stride floats from H1).
struct Partials {
    float* H1 = nullptr;
    int np = 0;
    int64_t stride = 0;
};

// GEMM2 into H, splitting K when the shape calls for it; the partials beyond the
// first go to `part` and are then either handed back (*out, for the combine to
// add) or folded into H.
moe_status gemm2_impl(const moe_dims& d, const void* h, const int32_t* offsets, const void* w_down, float* H,
                      void* tp, float* part, Partials* out, hipStream_t st, bool prefix_ready = false) {
    const int64_t R = max_rows(d);
    float* H1 = partial_bytes(d) ? part : nullptr;
    MOE_CHECK_HIP(launch_gemm2(d.dtype, h, offsets, d.E, R, w_down, H, H1, d.d, d.m, tp, st, prefix_ready,
                               group_rows(d)));
    const int np = H1 ? gemm2_splits(d.dtype, R, d.E, d.d, d.m, group_rows(d)) - 1 : 0;
    if (out) {
        out->H1 = H1;
        out->np = np;
        out->stride = R * d.d;
    } else if (np) {
        MOE_CHECK_HIP(launch_add_partial(H, H1, np, offsets, d.E, R, d.d, st));
    }
    return MOE_OK;
}

// prefix_ready: the tile prefix at the start of ws was written by the dispatch scan.
// gather (nullable): x_perm is then the token-ordered x, read through it (gather_rows)
moe_status ffn_impl(const moe_dims& d, const void* x_perm, const int32_t* offsets, const void* w_gate,
                    const void* w_up, const void* w_down, float* H, void* ws, Partials* out, hipStream_t st,
                    bool prefix_ready = false, const int32_t* gather = nullptr) {
    void* tp = ws;
    char* h = static_cast<char*>(ws) + align_up(gemm_ws_bytes(d.E));
    float* g1part = reinterpret_cast<float*>(h + align_up((size_t)max_rows(d) * d.m * elem(d)));
    float* part = reinterpret_cast<float*>(reinterpret_cast<char*>(g1part) + g1_part_bytes(d));
    const int64_t R = max_rows(d);
    MOE_CHECK_HIP(launch_gemm1(d.dtype, x_perm, offsets, d.E, R, w_gate, w_up, h, d.m, d.d, tp, st, prefix_ready,
                               g1_part_bytes(d) ? g1part : nullptr, gather, group_rows(d)));
    // GEMM2 uses the same row tiles: the prefix GEMM1 found (or was given) stays valid
    return gemm2_impl(d, h, offsets, w_down, H, tp, part, out, st, true);
}

moe_status shared_impl(const moe_dims& d, const void* x, const void* s_gate, const void* s_up, const void* s_down,
                       float* s, void* ws, hipStream_t st) {
    void* tp = ws;
    char* h = static_cast<char*>(ws) + align_up(gemm_ws_bytes(1));
    float* g1part = reinterpret_cast<float*>(h + align_up((size_t)d.T * d.m_shared * elem(d)));
    float* part = reinterpret_cast<float*>(reinterpret_cast<char*>(g1part) + shared_g1_bytes(d));
    MOE_CHECK_HIP(launch_gemm1(d.dtype, x, nullptr, 1, d.T, s_gate, s_up, h, d.m_shared, d.d, tp, st, false,
                               shared_g1_bytes(d) ? g1part : nullptr, nullptr, d.T));
    float* H1 = shared_g2_bytes(d) ? part : nullptr;
    MOE_CHECK_HIP(launch_gemm2(d.dtype, h, nullptr, 1, d.T, s_down, s, H1, d.d, d.m_shared, tp, st, false, d.T));
    if (H1) {
        const int np = gemm2_splits(d.dtype, d.T, 1, d.d, d.m_shared, d.T) - 1;
        MOE_CHECK_HIP(launch_add_partial(s, H1, np, nullptr, 1, d.T, d.d, st));
    }
    return MOE_OK;
}

}  // namespace

namespace {

// ---- the allocation-free forward's scratch -----------------------------------
// One workspace per device in a file-scope device array, zero when the module is
// loaded (the router's sync words at its start need that; every call leaves them
// at zero).  In host code `scratch` only names the symbol: its device address is
// looked up once per device, with that device current, and only that address is
// ever passed to kernels.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

hipError_t scratch_address(hipStream_t st, void** out) {
    hipDevice_t dev = 0;
    hipError_t e = hipStreamGetDevice(st, &dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t r = cur != dev ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess) return e;
        if (r != hipSuccess) return r;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

// The whole layer; side_ok: the shared expert may run on a side stream (else on
// the caller's stream, after the dispatch).
moe_status forward_impl(const moe_shape* shape, const void* x, const float* w_r, const float* b_r, const void* w_gate,
                        const void* w_up, const void* w_down, const void* s_gate, const void* s_up,
                        const void* s_down, float* y, int32_t* topk_ids, float* topk_w, int32_t* load, int32_t* slot,
                        int32_t* stats, int32_t* status, void* ws, size_t ws_bytes, void* stream, bool side_ok) {
    moe_dims d;
    moe_status rc = check_shape(shape, &d);
    if (rc != MOE_OK) return rc;
    if (!status || !load || !stats || !ws || !w_gate || !w_up || !w_down) return MOE_ERR_INVALID_ARGUMENT;
    if (d.T > 0 && (!x || !w_r || !y || !topk_ids || !topk_w || !slot)) return MOE_ERR_INVALID_ARGUMENT;
    if (d.m_shared && (!s_gate || !s_up || !s_down)) return MOE_ERR_INVALID_ARGUMENT;
    ForwardWs w = carve_forward(d, ws);
    if (ws_bytes < w.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
    hipStream_t st = static_cast<hipStream_t>(stream);
    // The shared expert runs on the caller stream's side stream, forked before
    // the front: its GEMMs then use CUs that the latency-bound router and
    // dispatch leave idle.  (Forked after the dispatch instead, the front is not
    // stretched, but the shared GEMMs then take CUs from the routed GEMM1 and the
    // DeepSeek-V3-like layer measured 0.7 % slower.)
    SideStream* side = nullptr;
    std::unique_lock<std::mutex> side_lock;
    bool side_forked = false;
    auto fork_shared = [&]() -> moe_status {
        if (!side_ok) return shared_impl(d, x, s_gate, s_up, s_down, w.s, w.shared, st);
        MOE_CHECK_HIP(side_stream(st, &side));
        side_lock = std::unique_lock<std::mutex>(side->mu);
        MOE_CHECK_HIP(hipEventRecord(side->fork, st));
        MOE_CHECK_HIP(hipStreamWaitEvent(side->stream, side->fork, 0));
        side_forked = true;
        const moe_status r = shared_impl(d, x, s_gate, s_up, s_down, w.s, w.shared, side->stream);
        if (hipEventRecord(side->join, side->stream) != hipSuccess) return MOE_ERR_HIP;
        return r;
    };
    // every return below first joins the side stream, also on an error
    auto joined = [&](moe_status r) -> moe_status {
        if (side_forked && hipStreamWaitEvent(st, side->join, 0) != hipSuccess) return MOE_ERR_HIP;
        return r;
    };
    const bool shared = d.m_shared && d.T > 0;
    // the dispatch (or the one-workgroup front of small batches) also writes the
    // GEMMs' tile prefix at the start of the FFN workspace
    int32_t* tprefix = static_cast<int32_t*>(w.ffn);
    if (shared && side_ok && (rc = fork_shared()) != MOE_OK) return joined(rc);
    if (front_fused_ok(d)) {
        if (launch_front(d, x, w_r, b_r, topk_ids, topk_w, status, w.route, st, load, w.offsets, slot, w.row_of,
                         w.src_token, w.x_perm, stats, tprefix, gemm_tile_rows(d.dtype)) != hipSuccess)
            return joined(MOE_ERR_HIP);
    } else {
        // where it can, the router also counts the dispatch's expert loads
        bool counted = false;
        if (launch_route(d, x, w_r, b_r, topk_ids, topk_w, status, w.route, w.sync, st, nullptr,
                         dispatch_router_counts_ok(d) ? static_cast<int32_t*>(w.dispatch) : nullptr, &counted,
                         stats + MOE_STAT_TOKENS_DROPPED) != hipSuccess)
            return joined(MOE_ERR_HIP);
        if (launch_dispatch(d, x, topk_ids, topk_w, load, w.offsets, slot, w.row_of, w.src_token, w.x_perm, stats,
                            w.dispatch, st, tprefix, gemm_tile_rows(d.dtype), counted, counted ? status : nullptr,
                            w.sync + 1) != hipSuccess)
            return joined(MOE_ERR_HIP);
    }
    // without a side stream the shared expert runs on `stream`, after the dispatch
    if (shared && !side_ok && (rc = fork_shared()) != MOE_OK) return joined(rc);
    Partials parts;   // K-split partials of H beyond the first, added by the combine
    rc = w.x_perm ? ffn_impl(d, w.x_perm, w.offsets, w_gate, w_up, w_down, w.H, w.ffn, &parts, st, true)
                  : ffn_impl(d, x, w.offsets, w_gate, w_up, w_down, w.H, w.ffn, &parts, st, true, w.src_token);
    rc = joined(rc);
    if (rc != MOE_OK) return rc;
    return hip_status(launch_combine(d, w.H, parts.H1, parts.np, parts.stride, w.row_of, topk_w, w.s, y, st));
}

}  // namespace

extern "C" {

int32_t moe_capacity(int64_t T, int32_t k, int32_t E, int32_t cf_num, int32_t cf_den) {
    if (T < 0 || k < 1 || E < 1 || cf_num < 1 || cf_den < 1) return -1;
    // ceil(cf_num * T * k / (cf_den * E)) without overflow for T < 2^31
    const __int128 num = (__int128)cf_num * T * k;
    const __int128 den = (__int128)cf_den * E;
    const __int128 c = (num + den - 1) / den;
    if (c > INT_MAX) return -1;
    return (int32_t)c;
}

moe_status moe_check_shape(const moe_shape* shape) { return check_shape(shape, nullptr); }

int64_t moe_max_rows(const moe_shape* shape) {
    moe_dims d;
    if (check_shape(shape, &d) != MOE_OK) return 0;
    return max_rows(d);
}

size_t moe_workspace_bytes(const moe_shape* shape, int32_t kind) {
    moe_dims d;
    if (check_shape(shape, &d) != MOE_OK) return 0;
    switch (kind) {
        case MOE_WS_ROUTE: return route_ws(d) + ALIGN;
        case MOE_WS_ROUTE_STATS: return route_stats_ws(d) + ALIGN;
        case MOE_WS_DISPATCH: return align_up(dispatch_ws_bytes(d)) + ALIGN;
        case MOE_WS_FFN: return ffn_ws(d);
        case MOE_WS_SHARED: return d.m_shared ? shared_ws(d) : 0;
        case MOE_WS_FORWARD: return carve_forward(d, nullptr).total;
        default: return 0;
    }
}

const char* moe_status_str(int32_t status) {
    switch (status) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT: bad shape, pointer, k or capacity";
        case MOE_ERR_NONFINITE_LOGIT: return "MOE_ERR_NONFINITE_LOGIT: a router score is NaN or infinite";
        case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: shape outside the supported range";
        case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP runtime call or kernel launch failed";
        default: return "unknown moe_status";
    }
}

moe_status moe_route_stats(const moe_shape* shape, const void* x, const float* w_r, const float* b_r,
                           int32_t* topk_ids, float* topk_w, int32_t* status, float* prob_sum, void* ws,
                           size_t ws_bytes, void* stream) {
    moe_dims d;
    moe_status rc = check_shape(shape, &d);
    if (rc != MOE_OK) return rc;
    if (!status || !prob_sum || (d.T > 0 && (!x || !w_r || !topk_ids || !topk_w))) return MOE_ERR_INVALID_ARGUMENT;
    if (!ws || ws_bytes < route_stats_ws(d)) return MOE_ERR_WORKSPACE_TOO_SMALL;
    hipStream_t st = static_cast<hipStream_t>(stream);
    char* base = static_cast<char*>(ws);
    float* probs = reinterpret_cast<float*>(base + route_ws(d));
    MOE_CHECK_HIP(launch_route(d, x, w_r, b_r, topk_ids, topk_w, status, base + MOE_SYNC_BYTES,
                               reinterpret_cast<int32_t*>(base), st, probs));
    return hip_status(launch_prob_sum(d, probs, prob_sum, st));
}

moe_status moe_pack_weights(const void* src, void* dst, int64_t batch, int64_t rows, int64_t cols,
                            int32_t elem_bytes, void* stream) {
    if (batch < 0 || rows < 0 || cols < 0 || (elem_bytes != 2 && elem_bytes != 4)) return MOE_ERR_INVALID_ARGUMENT;
    if (batch == 0 || rows == 0 || cols == 0) return MOE_OK;
    if (batch > 65535 || rows > 65535 * 64) return MOE_ERR_UNSUPPORTED;
    if (cols > INT64_MAX / 4 / batch / rows) return MOE_ERR_UNSUPPORTED;   // the byte count must fit int64
    if (!src || !dst) return MOE_ERR_INVALID_ARGUMENT;
    const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
    const uintptr_t n = static_cast<uintptr_t>(batch * rows * cols * elem_bytes);
    if (a < b + n && b < a + n) return MOE_ERR_INVALID_ARGUMENT;   // overlapping buffers
    return hip_status(launch_transpose(src, dst, batch, rows, cols, elem_bytes, static_cast<hipStream_t>(stream)));
}

moe_status moe_balance(const moe_shape* shape, const int32_t* load, const int32_t* stats, const float* prob_sum,
                       float* out, void* stream) {
    moe_dims d;
    moe_status rc = check_shape(shape, &d);
    if (rc != MOE_OK) return rc;
    if (!load || !stats || !prob_sum || !out) return MOE_ERR_INVALID_ARGUMENT;
    return hip_status(launch_balance(d, load, stats, prob_sum, out, static_cast<hipStream_t>(stream)));
}

moe_status moe_route(const moe_shape* shape, const void* x, const float* w_r, const float* b_r, int32_t* topk_ids,
                     float* topk_w, int32_t* status, void* ws, size_t ws_bytes, void* stream) {
    moe_dims d;
    moe_status rc = check_shape(shape, &d);
    if (rc != MOE_OK) return rc;
    if (!status || (d.T > 0 && (!x || !w_r || !topk_ids || !topk_w))) return MOE_ERR_INVALID_ARGUMENT;
    if (!ws || ws_bytes < route_ws(d)) return MOE_ERR_WORKSPACE_TOO_SMALL;
    char* base = static_cast<char*>(ws);
    return hip_status(launch_route(d, x, w_r, b_r, topk_ids, topk_w, status, base + MOE_SYNC_BYTES,
                                   reinterpret_cast<int32_t*>(base), static_cast<hipStream_t>(stream)));
}

moe_status moe_dispatch(const moe_shape* shape, const void* x, const int32_t* topk_ids, const float* topk_w,
                        int32_t* load, int32_t* offsets, int32_t* slot, int32_t* row_of, int32_t* src_token,
                        void* x_perm, int32_t* stats, void* ws, size_t ws_bytes, void* stream) {
    moe_dims d;
    moe_status rc = check_shape(shape, &d);
    if (rc != MOE_OK) return rc;
    if (!load || !offsets || !stats || !ws) return MOE_ERR_INVALID_ARGUMENT;
    if (d.T > 0 && (!x || !topk_ids || !slot || !row_of || !src_token || !x_perm)) return MOE_ERR_INVALID_ARGUMENT;
    if (d.T > 0 && d.accept_by_gate && !topk_w) return MOE_ERR_INVALID_ARGUMENT;
    if (ws_bytes < moe_workspace_bytes(shape, MOE_WS_DISPATCH)) return MOE_ERR_WORKSPACE_TOO_SMALL;
    return hip_status(launch_dispatch(d, x, topk_ids, topk_w, load, offsets, slot, row_of, src_token, x_perm, stats,
                                      ws, static_cast<hipStream_t>(stream)));
}

moe_status moe_expert_gemm1(const moe_shape* shape, const void* x_perm, const int32_t* offsets, const void* w_gate,
                            const void* w_up, void* h, void* ws, size_t ws_bytes, void* stream) {
    moe_dims d;
    moe_status rc = check_shape(shape, &d);
    if (rc != MOE_OK) return rc;
    if (!offsets || !ws || !w_gate || !w_up || (max_rows(d) > 0 && (!x_perm || !h))) return MOE_ERR_INVALID_ARGUMENT;
    if (ws_bytes < gemm1_ws(d)) return MOE_ERR_WORKSPACE_TOO_SMALL;
    float* g1part = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up(gemm_ws_bytes(d.E)));
    return hip_status(launch_gemm1(d.dtype, x_perm, offsets, d.E, max_rows(d), w_gate, w_up, h, d.m, d.d, ws,
                                   static_cast<hipStream_t>(stream), false, g1_part_bytes(d) ? g1part : nullptr,
                                   nullptr, group_rows(d)));
}

moe_status moe_expert_gemm2(const moe_shape* shape, const void* h, const int32_t* offsets, const void* w_down,
                            float* H, void* ws, size_t ws_bytes, void* stream) {
    moe_dims d;
    moe_status rc = check_shape(shape, &d);
    if (rc != MOE_OK) return rc;
    if (!offsets || !ws || !w_down || (max_rows(d) > 0 && (!h || !H))) return MOE_ERR_INVALID_ARGUMENT;
    if (ws_bytes < gemm2_ws(d)) return MOE_ERR_WORKSPACE_TOO_SMALL;
    float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up(gemm_ws_bytes(d.E)));
    return gemm2_impl(d, h, offsets, w_down, H, ws, part, nullptr, static_cast<hipStream_t>(stream));
}

moe_status moe_expert_ffn(const moe_shape* shape, const void* x_perm, const int32_t* offsets, const void* w_gate,
                          const void* w_up, const void* w_down, float* H, void* ws, size_t ws_bytes, void* stream) {
    moe_dims d;
    moe_status rc = check_shape(shape, &d);
    if (rc != MOE_OK) return rc;
    if (!offsets || !ws || !w_gate || !w_up || !w_down || (max_rows(d) > 0 && (!x_perm || !H)))
        return MOE_ERR_INVALID_ARGUMENT;
    if (ws_bytes < ffn_ws(d)) return MOE_ERR_WORKSPACE_TOO_SMALL;
    return ffn_impl(d, x_perm, offsets, w_gate, w_up, w_down, H, ws, nullptr, static_cast<hipStream_t>(stream));
}

moe_status moe_shared_ffn(const moe_shape* shape, const void* x, const void* s_gate, const void* s_up,
                          const void* s_down, float* s, void* ws, size_t ws_bytes, void* stream) {
    moe_dims d;
    moe_status rc = check_shape(shape, &d);
    if (rc != MOE_OK) return rc;
    if (d.m_shared == 0 || !s_gate || !s_up || !s_down || !ws || (d.T > 0 && (!x || !s)))
        return MOE_ERR_INVALID_ARGUMENT;
    if (ws_bytes < shared_ws(d)) return MOE_ERR_WORKSPACE_TOO_SMALL;
    return shared_impl(d, x, s_gate, s_up, s_down, s, ws, static_cast<hipStream_t>(stream));
}

moe_status moe_combine(const moe_shape* shape, const float* H, const int32_t* row_of, const float* topk_w,
                       const float* shared_out, float* y, void* stream) {
    moe_dims d;
    moe_status rc = check_shape(shape, &d);
    if (rc != MOE_OK) return rc;
    if (d.T > 0 && (!row_of || !topk_w || !y || (!H && max_rows(d) > 0))) return MOE_ERR_INVALID_ARGUMENT;
    return hip_status(
        launch_combine(d, H, nullptr, 0, 0, row_of, topk_w, shared_out, y, static_cast<hipStream_t>(stream)));
}

moe_status moe_forward(const moe_shape* shape, const void* x, const float* w_r, const float* b_r,
                       const void* w_gate, const void* w_up, const void* w_down, const void* s_gate,
                       const void* s_up, const void* s_down, float* y, int32_t* topk_ids, float* topk_w,
                       int32_t* load, int32_t* slot, int32_t* stats, int32_t* status, void* ws, size_t ws_bytes,
                       void* stream) {
    return forward_impl(shape, x, w_r, b_r, w_gate, w_up, w_down, s_gate, s_up, s_down, y, topk_ids, topk_w, load,
                        slot, stats, status, ws, ws_bytes, stream, true);
}

moe_status moe_forward_noalloc(const moe_shape* shape, const void* x, const float* w_r, const float* b_r,
                               const void* w_gate, const void* w_up, const void* w_down, const void* s_gate,
                               const void* s_up, const void* s_down, float* y, int32_t* topk_ids, float* topk_w,
                               int32_t* load, int32_t* slot, int32_t* stats, int32_t* status, void* stream) {
    moe_dims d;
    moe_status rc = check_shape(shape, &d);
    if (rc != MOE_OK) return rc;
    if (carve_forward(d, nullptr).total > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE_TOO_SMALL;
    void* ws = nullptr;
    if (scratch_address(static_cast<hipStream_t>(stream), &ws) != hipSuccess) return MOE_ERR_HIP;
    // the shared expert on the caller's stream: no side stream or event is made
    return forward_impl(shape, x, w_r, b_r, w_gate, w_up, w_down, s_gate, s_up, s_down, y, topk_ids, topk_w, load,
                        slot, stats, status, ws, MOE_NOALLOC_SCRATCH_BYTES, stream, false);
}

}  // extern "C"
