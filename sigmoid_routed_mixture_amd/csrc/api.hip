// The C ABI of include/moe.h: argument checks, workspace carving, stream/event orchestration, launches.
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "kernels.h"
#include "moe.h"
#include "moe_profile.h"
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

// Test knob: MOE_GEMM_PATH=wide|skinny forces one grouped-GEMM kernel for every size (both are exact
// implementations of the same GEMMs; the default picks by rows per expert).
moe::GemmPath pick_path(int T, int E, int k) {
    const char* f = std::getenv("MOE_GEMM_PATH");
    if (f && std::strcmp(f, "wide") == 0) return moe::GemmPath::Wide;
    if (f && std::strcmp(f, "skinny") == 0) return moe::GemmPath::Skinny;
    return moe::gemm_path(T, E, k);
}

} // namespace

namespace {

moe_status forward_impl(const moe_bf16* x, const moe_bf16* w_router, const float* bias, const moe_bf16* w1,
                        const moe_bf16* w3, const moe_bf16* w2, const moe_bf16* ws1, const moe_bf16* ws3,
                        const moe_bf16* ws2, int T, int H, int E, int k, int I, int Is, float scale, float* out,
                        int32_t* topk_ids, float* topk_gates, int32_t* expert_counts, void* workspace,
                        size_t workspace_bytes, void* stream, void* stream_shared, void* const* events) {
    g_last_error.clear();
    MOE_TRY(from_check(moe::check_sizes(T, H, E, k, I, Is, true)));
    if (T == 0) return MOE_OK;
    MOE_TRY(need(x, "x"));
    MOE_TRY(need(w_router, "w_router"));
    MOE_TRY(need(bias, "bias"));
    MOE_TRY(need(w1, "w1"));
    MOE_TRY(need(w3, "w3"));
    MOE_TRY(need(w2, "w2"));
    if (Is > 0) {
        MOE_TRY(need(ws1, "ws1"));
        MOE_TRY(need(ws3, "ws3"));
        MOE_TRY(need(ws2, "ws2"));
    }
    MOE_TRY(need(out, "out"));
    MOE_TRY(optional(topk_ids, "topk_ids"));
    MOE_TRY(optional(topk_gates, "topk_gates"));
    MOE_TRY(optional(expert_counts, "expert_counts"));
    if (workspace == nullptr) return fail(MOE_ERR_INVALID_ARG, "workspace is null");
    MOE_TRY(from_check(moe::check_aligned(workspace, "workspace", 256)));
    const moe::Layout L = moe::forward_layout(T, H, E, k, I, Is);
    if (workspace_bytes < L.total) return fail(MOE_ERR_WORKSPACE, "workspace smaller than moe_workspace_bytes");
    if (T == 0) return MOE_OK;

    char* ws = static_cast<char*>(workspace);
    auto at = [ws](size_t off) { return static_cast<void*>(ws + off); };
    int32_t* ids = topk_ids ? topk_ids : static_cast<int32_t*>(at(L.ids));
    float* gates = topk_gates ? topk_gates : static_cast<float*>(at(L.gates));
    int32_t* counts = expert_counts ? expert_counts : static_cast<int32_t*>(at(L.counts));
    int32_t* offsets = static_cast<int32_t*>(at(L.offsets));
    int32_t* row_token = static_cast<int32_t*>(at(L.row_token));
    int32_t* slot_row = static_cast<int32_t*>(at(L.slot_row));
    int2* tiles = static_cast<int2*>(at(L.tiles));
    int32_t* ntiles = static_cast<int32_t*>(at(L.ntiles));
    uint16_t* h_perm = static_cast<uint16_t*>(at(L.h_perm));
    float* y_perm = static_cast<float*>(at(L.y_perm));
    uint16_t* h_sh = Is > 0 ? static_cast<uint16_t*>(at(L.h_sh)) : nullptr;
    float* y_sh = Is > 0 ? static_cast<float*>(at(L.y_sh)) : nullptr;

    hipStream_t s0 = static_cast<hipStream_t>(stream);
    hipStream_t s1 = static_cast<hipStream_t>(stream_shared);
    const bool two_streams = Is > 0 && s1 != nullptr && s1 != s0;
    DeviceEvents* ev = nullptr;
    if (two_streams) MOE_TRY(device_events(&ev));

    const moe::GemmPath path = pick_path(T, E, k);
    const bool wide = path == moe::GemmPath::Wide;
    const int BM = wide ? moe::kWideBM : moe::kSkinnyBM;

    auto mark = [&](int i) -> moe_status {
        if (events == nullptr) return MOE_OK;
        return from_hip(hipEventRecord(static_cast<hipEvent_t>(events[i]), s0), "hipEventRecord (profile)");
    };
    MOE_TRY(mark(0));
    const int S = moe::router_splits(T, H);
    MOE_HIP(moe::launch_router(x, w_router, bias, T, H, E, k, scale, ids, gates, nullptr,
                               static_cast<float*>(at(L.partial)), S, s0),
            "router");
    MOE_TRY(mark(1));
    MOE_HIP(moe::launch_permute(ids, T, E, k, counts, offsets, row_token, slot_row,
                                static_cast<int32_t*>(at(L.chunk_base)), tiles, ntiles, BM, s0),
            "permute");
    MOE_TRY(mark(2));
    // The shared expert needs no routing: with a second stream it forks here, after the router and the
    // permutation (so it cannot delay them), and overlaps the routed experts.
    if (two_streams) MOE_TRY(order_after(s1, s0, ev->fork));
    if (Is > 0) {
        hipStream_t ss = two_streams ? s1 : s0;
        moe::GemmArgs g1{};
        g1.act = x;
        g1.w_a = ws1;
        g1.w_b = ws3;
        g1.out = h_sh;
        g1.dense_rows = T;
        g1.N = Is;
        g1.K = H;
        const int64_t dense_tiles = ((int64_t)T + BM - 1) / BM;
        MOE_HIP(moe::launch_gemm(moe::GemmKind::GateUp, wide, g1, dense_tiles, ss), "shared gate/up GEMM");
        moe::GemmArgs g2{};
        g2.act = h_sh;
        g2.w_a = ws2;
        g2.out = y_sh;
        g2.dense_rows = T;
        g2.N = H;
        g2.K = Is;
        MOE_HIP(moe::launch_gemm(moe::GemmKind::DownF32, wide, g2, dense_tiles, ss), "shared down GEMM");
    }
    MOE_TRY(mark(3));

    const int64_t grid_tiles = moe::max_tiles(T, E, k, BM);
    moe::GemmArgs r1{};
    r1.act = x;
    r1.row_token = row_token;
    r1.w_a = w1;
    r1.w_b = w3;
    r1.out = h_perm;
    r1.counts = counts;
    r1.offsets = offsets;
    r1.tiles = tiles;
    r1.ntiles = ntiles;
    r1.groups = E;
    r1.N = I;
    r1.K = H;
    MOE_HIP(moe::launch_gemm(moe::GemmKind::GateUp, wide, r1, grid_tiles, s0), "routed gate/up GEMM");
    MOE_TRY(mark(4));
    moe::GemmArgs r2{};
    r2.act = h_perm;
    r2.w_a = w2;
    r2.out = y_perm;
    r2.counts = counts;
    r2.offsets = offsets;
    r2.tiles = tiles;
    r2.ntiles = ntiles;
    r2.groups = E;
    r2.N = H;
    r2.K = I;
    MOE_HIP(moe::launch_gemm(moe::GemmKind::DownF32, wide, r2, grid_tiles, s0), "routed down GEMM");
    MOE_TRY(mark(5));

    if (two_streams) MOE_TRY(order_after(s0, s1, ev->join));
    MOE_HIP(moe::launch_combine(y_perm, gates, slot_row, y_sh, T, H, k, out, s0), "combine");
    MOE_TRY(mark(6));
    return MOE_OK;
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

size_t moe_workspace_bytes(int T, int H, int E, int k, int I, int Is) {
    if (!moe::check_sizes(T, H, E, k, I, Is, true).ok()) return 0;
    return moe::forward_layout(T, H, E, k, I, Is).total;
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
                                static_cast<int32_t*>(workspace), nullptr, nullptr, 0, s),
            "permute");
    if (x_perm) MOE_HIP(moe::launch_gather_rows(x, row_token, offsets, E, T, H, T * k, x_perm, s), "gather rows");
    return MOE_OK;
}

moe_status moe_forward(const moe_bf16* x, const moe_bf16* w_router, const float* bias, const moe_bf16* w1,
                       const moe_bf16* w3, const moe_bf16* w2, const moe_bf16* ws1, const moe_bf16* ws3,
                       const moe_bf16* ws2, int T, int H, int E, int k, int I, int Is, float scale, float* out,
                       int32_t* topk_ids, float* topk_gates, int32_t* expert_counts, void* workspace,
                       size_t workspace_bytes, void* stream, void* stream_shared) {
    return forward_impl(x, w_router, bias, w1, w3, w2, ws1, ws3, ws2, T, H, E, k, I, Is, scale, out, topk_ids,
                        topk_gates, expert_counts, workspace, workspace_bytes, stream, stream_shared, nullptr);
}

moe_status moe_forward_profiled(const moe_bf16* x, const moe_bf16* w_router, const float* bias,
                                const moe_bf16* w1, const moe_bf16* w3, const moe_bf16* w2, const moe_bf16* ws1,
                                const moe_bf16* ws3, const moe_bf16* ws2, int T, int H, int E, int k, int I, int Is,
                                float scale, float* out, int32_t* topk_ids, float* topk_gates,
                                int32_t* expert_counts, void* workspace, size_t workspace_bytes, void* stream,
                                void* stream_shared, void* const* events) {
    if (events == nullptr) return fail(MOE_ERR_INVALID_ARG, "events is null");
    for (int i = 0; i < 7; ++i)
        if (events[i] == nullptr) return fail(MOE_ERR_INVALID_ARG, "an event is null");
    return forward_impl(x, w_router, bias, w1, w3, w2, ws1, ws3, ws2, T, H, E, k, I, Is, scale, out, topk_ids,
                        topk_gates, expert_counts, workspace, workspace_bytes, stream, stream_shared, events);
}

} // extern "C"
