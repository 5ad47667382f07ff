// The C ABI of include/moe.h: argument checks, workspace carving, stream/event orchestration, launches.
#include <algorithm>
#include <atomic>
#include <cstring>
#include <mutex>
#include <string>

#include "kernels.h"
#include "moe.h"
#include "moe_block.h"
#include "moe_profile.h"
#include "moe_tuning.h"
#include "plan.h"

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status s, const std::string& msg) {
    g_last_error = msg;
    return s;
}

moe_status from_check(const moe::Check& c) { return c.ok() ? MOE_OK : fail(c.status, c.message); }

moe_status from_hip(hipError_t e, const char* what) {
    if (e == hipSuccess) return MOE_OK;
    return fail(MOE_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

#define MOE_TRY(expr)                         \
    do {                                      \
        const moe_status _s = (expr);         \
        if (_s != MOE_OK) return _s;          \
    } while (0)

#define MOE_HIP(expr, what) MOE_TRY(from_hip((expr), (what)))

moe_status need(const void* p, const char* name) {
    if (p == nullptr) return fail(MOE_ERR_INVALID_ARG, std::string(name) + " is null");
    return from_check(moe::check_aligned(p, name));
}

moe_status optional(const void* p, const char* name) {
    return p == nullptr ? MOE_OK : from_check(moe::check_aligned(p, name));
}

// One fork/join event pair per device for the shared-expert stream; the mutex makes each record + wait
// pair atomic with respect to other host threads using the same device.
struct DeviceEvents {
    std::once_flag once;
    hipError_t status = hipSuccess;
    hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int kMaxDevices = 64;
DeviceEvents g_events[kMaxDevices];
std::mutex g_event_mutex;

moe_status device_events(DeviceEvents** out) {
    int dev = 0;
    MOE_HIP(hipGetDevice(&dev), "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device index >= 64");
    DeviceEvents& d = g_events[dev];
    std::call_once(d.once, [&d]() {
        d.status = hipEventCreateWithFlags(&d.fork, hipEventDisableTiming);
        if (d.status == hipSuccess) d.status = hipEventCreateWithFlags(&d.join, hipEventDisableTiming);
    });
    MOE_HIP(d.status, "hipEventCreateWithFlags");
    *out = &d;
    return MOE_OK;
}

moe_status order_after(hipStream_t waiter, hipStream_t signaller, hipEvent_t ev) {
    std::lock_guard<std::mutex> lock(g_event_mutex);
    MOE_HIP(hipEventRecord(ev, signaller), "hipEventRecord");
    MOE_HIP(hipStreamWaitEvent(waiter, ev, 0), "hipStreamWaitEvent");
    return MOE_OK;
}

// Scratch of moe_forward_noalloc: the forward pass's workspace as file-scope device memory, one copy per
// device, held until the process ends. Host code never uses the array's name as an address (on the host it
// is only a stand-in): each device's address comes from hipGetSymbolAddress, taken once per device with
// that device current.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

struct DeviceScratch {
    std::once_flag once;
    hipError_t status = hipSuccess;
    void* ptr = nullptr;
};
DeviceScratch g_scratch[kMaxDevices];

moe_status device_scratch(void** out) {
    int dev = 0;
    MOE_HIP(hipGetDevice(&dev), "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device index >= 64");
    DeviceScratch& d = g_scratch[dev];
    std::call_once(d.once, [&d]() { d.status = hipGetSymbolAddress(&d.ptr, HIP_SYMBOL(scratch)); });
    MOE_HIP(d.status, "hipGetSymbolAddress (scratch)");
    if (d.ptr == nullptr) return fail(MOE_ERR_HIP, "hipGetSymbolAddress (scratch) returned null");
    *out = d.ptr;
    return MOE_OK;
}

// Overrides of the size rules (include/moe_tuning.h), read once per call: 0 everywhere unless a test or
// benchmark set one.
std::atomic<int> g_tuning[MOE_TUNE_KNOBS];
constexpr int kTuneMax[MOE_TUNE_KNOBS] = {4, 1, 1, 3, 4, 1, 3, 1, 2};

int tuning(moe_tune_knob k) { return g_tuning[k].load(std::memory_order_relaxed); }

// The GEMM kernel: gemm_path for the grouped GEMMs, dense_path for a dense MLP of T rows, unless the
// MOE_TUNE_GEMM_PATH knob forces one (all are exact implementations of the same GEMMs). The Dma kernel is
// used only when every operand fits its 32-bit offsets: x [T, H], h [T k + T, I] and [T, Is], the weights.
moe::GemmPath pick_path(int T, int E, int k, int H, int I, int Is, bool dense = false) {
    const bool fits = moe::dma_fits(T, H) && moe::dma_fits((int64_t)T * k + T, I) && moe::dma_fits(T, Is) &&
                      moe::dma_fits(I, H) && moe::dma_fits(H, I) && moe::dma_fits(Is, H) && moe::dma_fits(H, Is);
    moe::GemmPath p = dense ? moe::dense_path(T) : moe::gemm_path(T, E, k);
    switch (tuning(MOE_TUNE_GEMM_PATH)) {
    case 1: p = moe::GemmPath::Wide; break;
    case 2: p = moe::GemmPath::Tall; break;
    case 3: p = moe::GemmPath::Dma; break;
    case 4: p = moe::GemmPath::Skinny; break;
    default: break;
    }
    return p == moe::GemmPath::Dma && !fits ? moe::fallback_path(T, E, k) : p;
}

// A dense SwiGLU MLP (the shared expert, or the dense-first blocks' MLP): gate/up into h, then down into
// the fp32 out. On the weight-streaming kernel with few workgroups each GEMM splits K into fp32 partials
// (`part`, sized by dense_partial_bytes) reduced in split order.
moe_status dense_mlp(moe::GemmPath path, const uint16_t* x, const uint16_t* w1, const uint16_t* w3,
                     const uint16_t* w2, int T, int H, int I, uint16_t* h, float* out, float* part, hipStream_t s,
                     const char* what) {
    const int BM = moe::path_bm(path);
    const int64_t tiles = ((int64_t)T + BM - 1) / BM;
    const bool skinny = path == moe::GemmPath::Skinny;
    // few rows on the LDS-copy kernel: K split by the device's CU count (partials in `part`, then reduced)
    const bool dma_split = path == moe::GemmPath::Dma && T <= moe::kDmaSplitMaxT && part != nullptr;
    int cus = 0;
    if (dma_split) MOE_HIP(moe::device_cus(cus), "hipDeviceGetAttribute (compute units)");
    // up to 32 rows the deep copy ring: streamed (ring knobs 0 and 3) where the splits of both GEMMs can be
    // multiples of its 4-step period, else one workgroup per block (knob 2 forces that)
    const int ring = tuning(MOE_TUNE_RING);
    const int deep = path == moe::GemmPath::Dma && T <= moe::kDeepRingMaxT && ring != 1 ? (ring == 2 ? 1 : 2) : 0;
    int s1 = 1, s2 = 1;
    if (skinny && part) {
        s1 = moe::dense_splits(true, T, I, H);
        s2 = moe::dense_splits(false, T, H, I);
    } else if (dma_split) {
        const int t1 = deep == 2 ? moe::dma_stream_splits(true, T, I, H, cus) : 0;
        const int t2 = deep == 2 ? moe::dma_stream_splits(false, T, H, I, cus) : 0;
        s1 = t1 > 0 ? t1 : moe::dma_dense_splits(true, T, I, H, cus);
        s2 = t2 > 0 ? t2 : moe::dma_dense_splits(false, T, H, I, cus);
    }
    moe::GemmArgs g1{};
    g1.act = x;
    g1.w_a = w1;
    g1.w_b = w3;
    g1.out = s1 > 1 && skinny ? static_cast<void*>(part) : static_cast<void*>(h);
    g1.dense_rows = T;
    g1.N = I;
    g1.K = H;
    g1.ksplit = s1;
    g1.part = part;
    g1.part_rows = T;
    g1.deep = deep;
    const std::string w(what);
    MOE_HIP(moe::launch_gemm(moe::GemmKind::GateUp, path, g1, tiles, s), (w + " gate/up GEMM").c_str());
    if (s1 > 1) MOE_HIP(moe::launch_reduce(moe::GemmKind::GateUp, part, s1, T, I, h, s), (w + " gate/up reduce").c_str());
    moe::GemmArgs g2{};
    g2.act = h;
    g2.w_a = w2;
    g2.out = s2 > 1 && skinny ? static_cast<void*>(part) : static_cast<void*>(out);
    g2.dense_rows = T;
    g2.N = H;
    g2.K = I;
    g2.ksplit = s2;
    g2.part = part;
    g2.part_rows = T;
    g2.deep = g1.deep;
    MOE_HIP(moe::launch_gemm(moe::GemmKind::DownF32, path, g2, tiles, s), (w + " down GEMM").c_str());
    if (s2 > 1) MOE_HIP(moe::launch_reduce(moe::GemmKind::DownF32, part, s2, T, H, out, s), (w + " down reduce").c_str());
    return MOE_OK;
}

} // namespace

namespace {

// One mixture pass. The input is either x (the normalised stream) or resid + gamma (the block entry
// point normalises first and adds resid back in the combine); the routing is either computed (w_router,
// bias, scale) or given (ids_in, gates_in).
struct Request {
    const moe_bf16* x = nullptr;
    const moe_bf16* resid = nullptr;
    const moe_bf16* gamma = nullptr;
    double eps = 0.0;
    moe_bf16* x_norm = nullptr;
    const moe_bf16* w_router = nullptr;
    const float* bias = nullptr;
    float scale = 1.0f;
    const int32_t* ids_in = nullptr;
    const float* gates_in = nullptr;
    const moe_bf16 *w1 = nullptr, *w3 = nullptr, *w2 = nullptr, *ws1 = nullptr, *ws3 = nullptr, *ws2 = nullptr;
    int T = 0, H = 0, E = 0, k = 0, I = 0, Is = 0;
    float* out = nullptr;
    int32_t* topk_ids = nullptr;
    float* topk_gates = nullptr;
    int32_t* expert_counts = nullptr;
    void* workspace = nullptr;
    size_t workspace_bytes = 0;
    void* stream = nullptr;
    void* stream_shared = nullptr;
    void* const* events = nullptr;
};

moe_status forward_impl(const Request& q) {
    g_last_error.clear();
    const int T = q.T, H = q.H, E = q.E, k = q.k, I = q.I, Is = q.Is;
    const bool block = q.resid != nullptr || q.gamma != nullptr;
    const bool given = q.ids_in != nullptr || q.gates_in != nullptr;
    MOE_TRY(from_check(moe::check_sizes(T, H, E, k, I, Is, true)));
    if (block && !(q.eps >= 0.0 && q.eps <= 1e300)) return fail(MOE_ERR_INVALID_ARG, "eps is negative or not finite");
    if (T == 0) return MOE_OK;
    if (block) {
        MOE_TRY(need(q.resid, "resid"));
        MOE_TRY(need(q.gamma, "gamma"));
        MOE_TRY(optional(q.x_norm, "x_norm"));
    } else {
        MOE_TRY(need(q.x, "x"));
    }
    if (given) {
        MOE_TRY(need(q.ids_in, "topk_ids"));
        MOE_TRY(need(q.gates_in, "topk_gates"));
    } else {
        MOE_TRY(need(q.w_router, "w_router"));
        MOE_TRY(need(q.bias, "bias"));
        MOE_TRY(optional(q.topk_ids, "topk_ids"));
        MOE_TRY(optional(q.topk_gates, "topk_gates"));
    }
    MOE_TRY(need(q.w1, "w1"));
    MOE_TRY(need(q.w3, "w3"));
    MOE_TRY(need(q.w2, "w2"));
    if (Is > 0) {
        MOE_TRY(need(q.ws1, "ws1"));
        MOE_TRY(need(q.ws3, "ws3"));
        MOE_TRY(need(q.ws2, "ws2"));
    }
    MOE_TRY(need(q.out, "out"));
    MOE_TRY(optional(q.expert_counts, "expert_counts"));
    if (q.workspace == nullptr) return fail(MOE_ERR_INVALID_ARG, "workspace is null");
    MOE_TRY(from_check(moe::check_aligned(q.workspace, "workspace", 256)));
    const moe::Layout L = moe::forward_layout(T, H, E, k, I, Is, block);
    if (q.workspace_bytes < L.total)
        return fail(MOE_ERR_WORKSPACE, block ? "workspace smaller than moe_block_workspace_bytes"
                                             : "workspace smaller than moe_workspace_bytes");

    char* ws = static_cast<char*>(q.workspace);
    auto at = [ws](size_t off) { return static_cast<void*>(ws + off); };
    const int32_t* ids;
    const float* gates;
    int32_t* ids_out = nullptr;
    float* gates_out = nullptr;
    if (given) {
        ids = q.ids_in;
        gates = q.gates_in;
    } else {
        ids_out = q.topk_ids ? q.topk_ids : static_cast<int32_t*>(at(L.ids));
        gates_out = q.topk_gates ? q.topk_gates : static_cast<float*>(at(L.gates));
        ids = ids_out;
        gates = gates_out;
    }
    int32_t* counts = q.expert_counts ? q.expert_counts : static_cast<int32_t*>(at(L.counts));
    int32_t* offsets = static_cast<int32_t*>(at(L.offsets));
    int32_t* row_token = static_cast<int32_t*>(at(L.row_token));
    int32_t* slot_row = static_cast<int32_t*>(at(L.slot_row));
    int4* tiles = static_cast<int4*>(at(L.tiles));
    int32_t* ntiles = static_cast<int32_t*>(at(L.ntiles));
    uint16_t* h_perm = static_cast<uint16_t*>(at(L.h_perm));
    float* y_perm = static_cast<float*>(at(L.y_perm)); // per-slot rows, fp32 or bf16 (slot_rows_bf16)
    const moe::GemmPath path = pick_path(T, E, k, H, I, Is);
    const int BM = moe::path_bm(path);
    hipStream_t s0 = static_cast<hipStream_t>(q.stream);
    hipStream_t s1 = static_cast<hipStream_t>(q.stream_shared);
    const bool own_stream = s1 != nullptr && s1 != s0;
    // the shared expert at decode sizes: one more group of the routed GEMMs (rows T * k onwards of h_perm and
    // y_perm) when it has the routed width
    const bool fold = moe::shared_fold(T, E, k, I, Is);
    // the DMA kernel's work-balanced XCD split (computed for both grouped GEMMs, used by the down GEMM)
    const bool balanced = path == moe::GemmPath::Dma && !fold && tuning(MOE_TUNE_XCD_SPLIT) == 0;
    // the grouped DMA GEMMs run persistent (one workgroup per CU claiming blocks from per-XCD counters)
    const bool persist = balanced && tuning(MOE_TUNE_PERSIST) == 0;
    // above the decode sizes, with the routed width and no stream of its own: one more group of the persistent
    // routed GEMMs, its tiles spread over the XCDs, its fp32 rows in y_shared; else a dense MLP
    const bool fold_pre = persist && moe::shared_fold_prefill(T, E, k, I, Is) && !own_stream &&
                          tuning(MOE_TUNE_SHARED) == 0;
    const bool grouped_shared = fold || fold_pre;
    const bool dense_shared = Is > 0 && !grouped_shared;
    uint16_t* h_sh = nullptr;
    if (dense_shared) // its h: the rows after the routed ones when it has their width
        h_sh = Is == I ? h_perm + (size_t)T * k * I : static_cast<uint16_t*>(at(L.h_sh));
    float* y_sh = Is > 0 && !fold ? static_cast<float*>(at(L.y_sh)) : nullptr;
    if (fold) y_sh = y_perm + (size_t)T * k * H;
    const bool two_streams = dense_shared && own_stream;
    DeviceEvents* ev = nullptr;
    if (two_streams) MOE_TRY(device_events(&ev));

    auto mark = [&](int i) -> moe_status {
        if (q.events == nullptr || q.events[i] == nullptr) return MOE_OK;
        return from_hip(hipEventRecord(static_cast<hipEvent_t>(q.events[i]), s0), "hipEventRecord (profile)");
    };
    MOE_TRY(mark(0));
    // the mixture's input: x, or RMSNorm(resid) written to the caller's x_norm or the workspace
    const uint16_t* xin = q.x;
    if (block) {
        uint16_t* xn = q.x_norm ? q.x_norm : static_cast<uint16_t*>(at(L.x_norm));
        MOE_HIP(moe::launch_rmsnorm(q.resid, q.gamma, q.eps, T, H, xn, s0), "rmsnorm");
        xin = xn;
    }
    // up to kRouterSmallT tokens the router's top-k and the permutation share one launch (its ticket: the
    // first int of the permutation's chunk scratch, which a single chunk does not use)
    const int router_S = moe::router_splits(T, H, E);
    const bool route_permute = !given && T <= moe::kRouterSmallT && tuning(MOE_TUNE_ROUTE_PERMUTE) == 0;
    int32_t* ticket = route_permute ? static_cast<int32_t*>(at(L.chunk_base)) : nullptr;
    if (route_permute)
        MOE_HIP(moe::launch_router_logits_small(xin, q.w_router, T, H, E, static_cast<float*>(at(L.partial)),
                                                router_S, ticket, s0),
                "router logits");
    else if (!given)
        MOE_HIP(moe::launch_router(xin, q.w_router, q.bias, T, H, E, k, q.scale, ids_out, gates_out, nullptr,
                                   static_cast<float*>(at(L.partial)), router_S, s0),
                "router");
    MOE_TRY(mark(1));
    const int64_t grid_tiles = moe::max_tiles(T, E, k, BM) + (grouped_shared ? moe::shared_tiles(T, BM) : 0);
    moe::XcdSplit split{};
    if (balanced) {
        split.bounds = static_cast<int32_t*>(at(L.xcd_bounds));
        split.ntn[0] = moe::dma_ntn(true, I);
        split.ntn[1] = moe::dma_ntn(false, H);
        for (int v = 0; v < 2; ++v) split.cap[v] = (int)moe::dma_xcd_cap(grid_tiles, split.ntn[v]);
    }
    if (persist) split.ctr = static_cast<int32_t*>(at(L.xcd_bounds)) + 2 * (moe::kXcds + 1);
    // block order of the persistent GEMMs: experts in index order, each cut into chunks of at most
    // kPlainChunkTiles tiles (the MOE_TUNE_ORDER knob picks the longer chunks or one of the dealt orders)
    const int order = tuning(MOE_TUNE_ORDER);
    const bool dealt = persist && order >= 2;
    split.dealt = dealt ? order - 1 : 0;
    split.plain_cap = order == 1 ? moe::kMaxChunkTiles : moe::kPlainChunkTiles;
    split.spread_shared = fold_pre ? 1 : 0;
    int cus = 0;
    MOE_HIP(moe::device_cus(cus), "hipDeviceGetAttribute (compute units)");
    // experts (with the folded shared expert) a batch of this size is expected to reach
    const int64_t expect_groups = moe::expected_active(T, E, k) + (grouped_shared ? 1 : 0);
    // decode sizes: the deeper copy ring, streamed (one workgroup per CU, blocks back to back) where the launch
    // allows it and few blocks per CU are expected, else one workgroup per block (ring knob 2 forces that,
    // ring knob 3 the streamed form wherever the launch allows it)
    const int ring = tuning(MOE_TUNE_RING);
    const bool deep = path == moe::GemmPath::Dma && !persist && T <= moe::kDeepRingMaxT && ring != 1;
    auto deep_mode = [&](int ntn) {
        if (!deep) return 0;
        return ring == 3 || (ring == 0 && moe::decode_streamed(expect_groups * ntn, cus)) ? 2 : 1;
    };
    const int deep_gate_up = deep_mode(moe::dma_ntn(true, I)), deep_down = deep_mode(moe::dma_ntn(false, H));
    // decode-sized grouped GEMMs: the permutation picks each one's K split from the live block count, gate/up
    // 1 or 2, down 1 up to down_split_max(T), splits beyond two only into whole ring periods of 4 K steps (so
    // the streamed kernel can take them, and every copy ring computes the same split)
    const int ks_knob = tuning(MOE_TUNE_KSPLIT);
    const bool ks_off = ks_knob == 1, ks_on = ks_knob >= 2;
    const bool ksplit = path == moe::GemmPath::Dma && L.ks_flag != size_t(-1) && !ks_off;
    int32_t* ks_flag = ksplit ? static_cast<int32_t*>(at(L.ks_flag)) : nullptr;
    bool ks_gate_up = false; // the gate/up split needs a reduction launch: skipped when it can never pay
    int down_allow = 0;
    if (ksplit) {
        const int nk2 = I / 64;
        for (int S = 2; S <= moe::down_split_max(T) && S <= nk2; ++S)
            if (S == 2 || (nk2 % S == 0 && (nk2 / S) % 4 == 0)) down_allow |= 1 << S;
        // splits beyond two only where the rule would take one at the expected block count (a one-workgroup-
        // per-block launch is sized for the largest allowed split: its surplus workgroups still cost dispatches)
        if (ks_knob != 3 && moe::decode_ksplit_down(expect_groups * moe::dma_ntn(false, H), cus, down_allow) <= 2)
            down_allow &= 1 << 2;
        split.ksplit = ks_flag;
        split.ks_ntn[0] = moe::dma_ntn(true, I);
        split.ks_ntn[1] = moe::dma_ntn(false, H);
        const int nk1 = H / 64; // gate/up: two ranges, or four where they are whole ring periods
        split.ks_allow[0] = (1 << 2) | (nk1 % 4 == 0 && (nk1 / 4) % 4 == 0 ? 1 << 4 : 0);
        split.ks_allow[1] = down_allow;
        split.cus = cus;
        split.ks_force = ks_on ? ks_knob : 0;
        // the gate/up split needs a reduction launch: only when the experts the batch is expected to reach
        // would split (the down GEMM's planes are added by the combine, with no launch of their own).
        // Stream-K only in streamed launches: the down GEMM's by default, the gate/up GEMM's with knob value 2
        // (and then only with its reduction enqueued): it pays for neither the reduction nor the partials
        // there (plan.h, decode_streamk)
        const int64_t expect = (moe::expected_active(T, E, k) + moe::shared_tiles(T, BM)) * split.ks_ntn[0];
        const int sk_knob = ks_on ? 1 : tuning(MOE_TUNE_STREAMK);
        ks_gate_up = ks_on || moe::decode_ksplit(expect, cus) == 2 ||
                     (sk_knob == 2 && deep_gate_up == 2 && moe::decode_streamk(expect, cus));
        split.ks_streamk[0] = sk_knob == 2 && deep_gate_up == 2 && ks_gate_up ? 1 : 0;
        split.ks_streamk[1] = sk_knob != 1 && deep_down == 2 ? 1 : 0;
    }
    if (route_permute)
        MOE_HIP(moe::launch_route_permute_few(static_cast<const float*>(at(L.partial)), router_S, q.bias, T, E, k,
                                              q.scale, ids_out, gates_out, nullptr, ticket, counts, offsets, row_token,
                                              slot_row, tiles, ntiles, BM, grouped_shared ? T : 0, split, s0),
                "route and permute");
    else
        MOE_HIP(moe::launch_permute(ids, T, E, k, counts, offsets, row_token, slot_row,
                                    static_cast<int32_t*>(at(L.chunk_base)), tiles, ntiles, BM, grouped_shared ? T : 0,
                                    split, s0),
                "permute");
    MOE_TRY(mark(2));
    // The shared expert needs no routing: with a second stream it forks here, after the router and the
    // permutation (so it cannot delay them), and overlaps the routed experts.
    if (two_streams) MOE_TRY(order_after(s1, s0, ev->fork));
    if (dense_shared) {
        hipStream_t ss = two_streams ? s1 : s0;
        float* part = L.sh_partial != size_t(-1) ? static_cast<float*>(at(L.sh_partial)) : nullptr;
        const moe::GemmPath spath = pick_path(T, 1, 1, H, Is, 0, true);
        MOE_TRY(dense_mlp(spath, xin, q.ws1, q.ws3, q.ws2, T, H, Is, h_sh, y_sh, part, ss, "shared"));
    }
    MOE_TRY(mark(3));

    auto add_shared = [&](moe::GemmArgs& a, const moe_bf16* wa, const moe_bf16* wb) {
        if (!grouped_shared) return;
        a.ws_a = wa;
        a.ws_b = wb;
        a.shared_rows = T;
        a.shared_off = T * k;
    };
    moe::GemmArgs r1{};
    r1.act = xin;
    r1.row_token = row_token;
    r1.w_a = q.w1;
    r1.w_b = q.w3;
    r1.out = h_perm;
    r1.counts = counts;
    r1.offsets = offsets;
    r1.tiles = tiles;
    r1.ntiles = ntiles;
    r1.groups = E;
    r1.N = I;
    r1.K = H;
    // gate/up keeps the block-count split: its long weight stream makes blocks of any height cost about the
    // same (the work-balanced split measured 2 % slower there, 2 % faster on the down GEMM)
    add_shared(r1, q.ws1, q.ws3);
    if (persist) r1.work_ctr = reinterpret_cast<unsigned long long*>(split.ctr);
    if (dealt) r1.xcd_bounds = split.bounds;
    const int h_rows = T * k + (grouped_shared ? T : 0);
    if (ks_gate_up) {
        r1.ksplit_dev = ks_flag;
        r1.ks_allow = split.ks_allow[0];
        r1.part = static_cast<float*>(at(L.ks_part));
        r1.part_rows = h_rows;
    }
    r1.deep = deep_gate_up;
    r1.rt_rows = T * k;
    MOE_HIP(moe::launch_gemm(moe::GemmKind::GateUp, path, r1, grid_tiles, s0), "routed gate/up GEMM");
    if (ks_gate_up)
        MOE_HIP(moe::launch_reduce_ksplit(r1.part, ks_flag, h_rows, I, h_perm, s0), "gate/up K-split reduction");
    MOE_TRY(mark(4));
    moe::GemmArgs r2{};
    r2.act = h_perm;
    r2.w_a = q.w2;
    r2.out = y_perm;
    r2.counts = counts;
    r2.offsets = offsets;
    r2.tiles = tiles;
    r2.ntiles = ntiles;
    r2.groups = E;
    r2.N = H;
    r2.K = I;
    r2.xcd_bounds = balanced ? split.bounds + (moe::kXcds + 1) : nullptr;
    r2.work_ctr = persist ? reinterpret_cast<unsigned long long*>(split.ctr) + moe::kXcds : nullptr;
    float* y2 = ksplit ? static_cast<float*>(at(L.ks_part_down)) : nullptr;
    if (ksplit) {
        r2.ksplit_dev = ks_flag + 1;
        r2.ks_allow = down_allow;
        r2.part = y2;
        r2.part_rows = h_rows;
    }
    add_shared(r2, q.ws2, nullptr);
    const bool ybf = moe::slot_rows_bf16(T, E, k, I, Is) && !ksplit;
    r2.out_bf16 = ybf ? 1 : 0;
    if (fold_pre) r2.out_shared = y_sh;
    r2.deep = deep_down;
    MOE_HIP(moe::launch_gemm(moe::GemmKind::DownF32, path, r2, grid_tiles, s0), "routed down GEMM");
    MOE_TRY(mark(5));

    if (two_streams) MOE_TRY(order_after(s0, s1, ev->join));
    MOE_HIP(moe::launch_combine(y_perm, ybf, gates, slot_row, y_sh, block ? q.resid : nullptr, T, H, k, q.out,
                                s0, y2, y2 != nullptr && fold ? y2 + (size_t)T * k * H : nullptr,
                                ksplit ? ks_flag + 1 : nullptr, (size_t)h_rows * H),
            "combine");
    MOE_TRY(mark(6));
    return MOE_OK;
}

Request plain_request(const moe_bf16* x, const moe_bf16* w_router, const float* bias, const moe_bf16* w1,
                      const moe_bf16* w3, const moe_bf16* w2, const moe_bf16* ws1, const moe_bf16* ws3,
                      const moe_bf16* ws2, int T, int H, int E, int k, int I, int Is, float scale, float* out,
                      int32_t* topk_ids, float* topk_gates, int32_t* expert_counts, void* workspace,
                      size_t workspace_bytes, void* stream, void* stream_shared) {
    Request q;
    q.x = x;
    q.w_router = w_router;
    q.bias = bias;
    q.w1 = w1;
    q.w3 = w3;
    q.w2 = w2;
    q.ws1 = ws1;
    q.ws3 = ws3;
    q.ws2 = ws2;
    q.T = T;
    q.H = H;
    q.E = E;
    q.k = k;
    q.I = I;
    q.Is = Is;
    q.scale = scale;
    q.out = out;
    q.topk_ids = topk_ids;
    q.topk_gates = topk_gates;
    q.expert_counts = expert_counts;
    q.workspace = workspace;
    q.workspace_bytes = workspace_bytes;
    q.stream = stream;
    q.stream_shared = stream_shared;
    return q;
}

} // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
    switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported size";
    case MOE_ERR_MISALIGNED: return "misaligned pointer";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP error";
    }
    return "unknown status";
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

moe_status moe_set_tuning(int knob, int value) {
    g_last_error.clear();
    if (knob < 0 || knob >= MOE_TUNE_KNOBS) return fail(MOE_ERR_INVALID_ARG, "unknown tuning knob");
    if (value < 0 || value > kTuneMax[knob]) return fail(MOE_ERR_INVALID_ARG, "tuning value out of range");
    g_tuning[knob].store(value, std::memory_order_relaxed);
    return MOE_OK;
}

int moe_get_tuning(int knob) {
    if (knob < 0 || knob >= MOE_TUNE_KNOBS) return -1;
    return g_tuning[knob].load(std::memory_order_relaxed);
}

size_t moe_workspace_bytes(int T, int H, int E, int k, int I, int Is) {
    if (!moe::check_sizes(T, H, E, k, I, Is, true).ok()) return 0;
    return moe::forward_workspace_bound(T, H, E, k, I, Is);
}

size_t moe_permute_workspace_bytes(int T, int E) {
    if (T < 0 || E <= 0 || E > moe::kMaxE) return 0;
    return moe::permute_scratch_bytes(T, E);
}

moe_status moe_route(const moe_bf16* x, const moe_bf16* w_router, const float* bias, int T, int H, int E, int k,
                     float scale, int32_t* topk_ids, float* topk_gates, float* logits, void* stream) {
    g_last_error.clear();
    MOE_TRY(from_check(moe::check_sizes(T, H, E, k, 0, 0, false)));
    if (T == 0) return MOE_OK;
    MOE_TRY(need(x, "x"));
    MOE_TRY(need(w_router, "w_router"));
    MOE_TRY(need(bias, "bias"));
    MOE_TRY(need(topk_ids, "topk_ids"));
    MOE_TRY(need(topk_gates, "topk_gates"));
    MOE_TRY(optional(logits, "logits"));
    if (T == 0) return MOE_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    MOE_HIP(moe::launch_router(x, w_router, bias, T, H, E, k, scale, topk_ids, topk_gates, logits, nullptr, 1, s),
            "router");
    return MOE_OK;
}

moe_status moe_permute(const moe_bf16* x, const int32_t* topk_ids, int T, int H, int E, int k, int32_t* counts,
                       int32_t* offsets, int32_t* row_token, int32_t* slot_row, moe_bf16* x_perm, void* workspace,
                       size_t workspace_bytes, void* stream) {
    g_last_error.clear();
    MOE_TRY(from_check(moe::check_sizes(T, H, E, k, 0, 0, false)));
    if (T == 0) return MOE_OK;
    MOE_TRY(need(topk_ids, "topk_ids"));
    MOE_TRY(need(counts, "counts"));
    MOE_TRY(need(offsets, "offsets"));
    MOE_TRY(need(row_token, "row_token"));
    MOE_TRY(need(slot_row, "slot_row"));
    MOE_TRY(optional(x_perm, "x_perm"));
    if (x_perm) MOE_TRY(need(x, "x"));
    if (workspace == nullptr) return fail(MOE_ERR_INVALID_ARG, "workspace is null");
    MOE_TRY(from_check(moe::check_aligned(workspace, "workspace", 256)));
    if (workspace_bytes < moe::permute_scratch_bytes(T, E))
        return fail(MOE_ERR_WORKSPACE, "workspace smaller than moe_permute_workspace_bytes");
    if (T == 0) return MOE_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    MOE_HIP(moe::launch_permute(topk_ids, T, E, k, counts, offsets, row_token, slot_row,
                                static_cast<int32_t*>(workspace), nullptr, nullptr, 0, 0, moe::XcdSplit{}, s),
            "permute");
    if (x_perm) MOE_HIP(moe::launch_gather_rows(x, row_token, offsets, E, T, H, T * k, x_perm, s), "gather rows");
    return MOE_OK;
}

moe_status moe_forward(const moe_bf16* x, const moe_bf16* w_router, const float* bias, const moe_bf16* w1,
                       const moe_bf16* w3, const moe_bf16* w2, const moe_bf16* ws1, const moe_bf16* ws3,
                       const moe_bf16* ws2, int T, int H, int E, int k, int I, int Is, float scale, float* out,
                       int32_t* topk_ids, float* topk_gates, int32_t* expert_counts, void* workspace,
                       size_t workspace_bytes, void* stream, void* stream_shared) {
    return forward_impl(plain_request(x, w_router, bias, w1, w3, w2, ws1, ws3, ws2, T, H, E, k, I, Is, scale, out,
                                      topk_ids, topk_gates, expert_counts, workspace, workspace_bytes, stream,
                                      stream_shared));
}

moe_status moe_forward_routed(const moe_bf16* x, const int32_t* topk_ids, const float* topk_gates,
                              const moe_bf16* w1, const moe_bf16* w3, const moe_bf16* w2, const moe_bf16* ws1,
                              const moe_bf16* ws3, const moe_bf16* ws2, int T, int H, int E, int k, int I, int Is,
                              float* out, int32_t* expert_counts, void* workspace, size_t workspace_bytes,
                              void* stream, void* stream_shared) {
    Request q = plain_request(x, nullptr, nullptr, w1, w3, w2, ws1, ws3, ws2, T, H, E, k, I, Is, 1.0f, out,
                              nullptr, nullptr, expert_counts, workspace, workspace_bytes, stream, stream_shared);
    q.ids_in = topk_ids;
    q.gates_in = topk_gates;
    if (T > 0 && (topk_ids == nullptr || topk_gates == nullptr)) {
        g_last_error.clear();
        return fail(MOE_ERR_INVALID_ARG, topk_ids == nullptr ? "topk_ids is null" : "topk_gates is null");
    }
    return forward_impl(q);
}

size_t moe_block_workspace_bytes(int T, int H, int E, int k, int I, int Is) {
    if (!moe::check_sizes(T, H, E, k, I, Is, true).ok()) return 0;
    return moe::forward_workspace_bound(T, H, E, k, I, Is, true);
}

moe_status moe_block_forward(const moe_bf16* resid, const moe_bf16* gamma, double eps, const moe_bf16* w_router,
                             const float* bias, const moe_bf16* w1, const moe_bf16* w3, const moe_bf16* w2,
                             const moe_bf16* ws1, const moe_bf16* ws3, const moe_bf16* ws2, int T, int H, int E,
                             int k, int I, int Is, float scale, float* out, moe_bf16* x_norm, int32_t* topk_ids,
                             float* topk_gates, int32_t* expert_counts, void* workspace, size_t workspace_bytes,
                             void* stream, void* stream_shared) {
    Request q = plain_request(nullptr, w_router, bias, w1, w3, w2, ws1, ws3, ws2, T, H, E, k, I, Is, scale, out,
                              topk_ids, topk_gates, expert_counts, workspace, workspace_bytes, stream, stream_shared);
    q.resid = resid;
    q.gamma = gamma;
    q.eps = eps;
    q.x_norm = x_norm;
    if (T > 0 && (resid == nullptr || gamma == nullptr)) {
        g_last_error.clear();
        return fail(MOE_ERR_INVALID_ARG, resid == nullptr ? "resid is null" : "gamma is null");
    }
    return forward_impl(q);
}

size_t moe_dense_mlp_workspace_bytes(int T, int H, int I) {
    if (!moe::check_dense_sizes(T, H, I).ok()) return 0;
    return moe::dense_workspace_bound(T, H, I);
}

moe_status moe_dense_mlp(const moe_bf16* x, const moe_bf16* w1, const moe_bf16* w3, const moe_bf16* w2, int T,
                         int H, int I, float* out, void* workspace, size_t workspace_bytes, void* stream) {
    g_last_error.clear();
    MOE_TRY(from_check(moe::check_dense_sizes(T, H, I)));
    if (T == 0) return MOE_OK;
    MOE_TRY(need(x, "x"));
    MOE_TRY(need(w1, "w1"));
    MOE_TRY(need(w3, "w3"));
    MOE_TRY(need(w2, "w2"));
    MOE_TRY(need(out, "out"));
    if (workspace == nullptr) return fail(MOE_ERR_INVALID_ARG, "workspace is null");
    MOE_TRY(from_check(moe::check_aligned(workspace, "workspace", 256)));
    if (workspace_bytes < moe::dense_workspace_bytes(T, H, I))
        return fail(MOE_ERR_WORKSPACE, "workspace smaller than moe_dense_mlp_workspace_bytes");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const moe::GemmPath path = pick_path(T, 1, 1, H, I, 0, true);
    char* ws = static_cast<char*>(workspace);
    const size_t hbytes = ((size_t)T * (size_t)I * 2 + 255) / 256 * 256;
    float* part = moe::dense_partial_bytes(T, H, I) > 0 ? reinterpret_cast<float*>(ws + hbytes) : nullptr;
    MOE_TRY(dense_mlp(path, x, w1, w3, w2, T, H, I, reinterpret_cast<uint16_t*>(ws), out, part, s, "dense"));
    return MOE_OK;
}

size_t moe_forward_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

moe_status moe_forward_noalloc(const moe_bf16* x, const moe_bf16* w_router, const float* bias, const moe_bf16* w1,
                               const moe_bf16* w3, const moe_bf16* w2, const moe_bf16* ws1, const moe_bf16* ws3,
                               const moe_bf16* ws2, int T, int H, int E, int k, int I, int Is, float scale,
                               float* out, int32_t* topk_ids, float* topk_gates, int32_t* expert_counts,
                               void* stream) {
    g_last_error.clear();
    MOE_TRY(from_check(moe::check_sizes(T, H, E, k, I, Is, true)));
    if (T == 0) return MOE_OK;
    const size_t need = moe::forward_layout(T, H, E, k, I, Is).total;
    if (need > kNoAllocScratchBytes)
        return fail(MOE_ERR_WORKSPACE, "moe_forward_noalloc: these sizes need " + std::to_string(need) +
                                           " bytes of scratch, above its " + std::to_string(kNoAllocScratchBytes) +
                                           "-byte maximum (use moe_forward with a caller workspace)");
    void* ws = nullptr;
    MOE_TRY(device_scratch(&ws));
    // the same pass as moe_forward on the device's scratch (the shared expert on `stream`); every buffer
    // of that pass that must start at zero (the persistent GEMMs' block counters) is cleared by its kernels
    return forward_impl(plain_request(x, w_router, bias, w1, w3, w2, ws1, ws3, ws2, T, H, E, k, I, Is, scale, out,
                                      topk_ids, topk_gates, expert_counts, ws, kNoAllocScratchBytes, stream,
                                      nullptr));
}

moe_status moe_forward_profiled(const moe_bf16* x, const moe_bf16* w_router, const float* bias,
                                const moe_bf16* w1, const moe_bf16* w3, const moe_bf16* w2, const moe_bf16* ws1,
                                const moe_bf16* ws3, const moe_bf16* ws2, int T, int H, int E, int k, int I, int Is,
                                float scale, float* out, int32_t* topk_ids, float* topk_gates,
                                int32_t* expert_counts, void* workspace, size_t workspace_bytes, void* stream,
                                void* stream_shared, void* const* events) {
    if (events == nullptr) return fail(MOE_ERR_INVALID_ARG, "events is null");
    Request q = plain_request(x, w_router, bias, w1, w3, w2, ws1, ws3, ws2, T, H, E, k, I, Is, scale, out, topk_ids,
                              topk_gates, expert_counts, workspace, workspace_bytes, stream, stream_shared);
    q.events = events;
    return forward_impl(q);
}

} // extern "C"
