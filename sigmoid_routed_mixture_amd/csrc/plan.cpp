// Host-side argument checks, launch planning and workspace layout (no HIP dependency).
#include "plan.h"

#include <algorithm>
#include <cmath>

namespace moe {

namespace {
Check fail(moe_status s, std::string m) { return Check{s, std::move(m)}; }
size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
} // namespace

Check check_sizes(int T, int H, int E, int k, int I, int Is, bool need_I) {
    if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T < 0");
    if (H <= 0) return fail(MOE_ERR_INVALID_ARG, "H <= 0");
    if (E <= 0) return fail(MOE_ERR_INVALID_ARG, "E <= 0");
    if (k < 1) return fail(MOE_ERR_INVALID_ARG, "k < 1");
    if (k > E) return fail(MOE_ERR_INVALID_ARG, "k > E");
    if (need_I && I <= 0) return fail(MOE_ERR_INVALID_ARG, "I <= 0");
    if (need_I && Is < 0) return fail(MOE_ERR_INVALID_ARG, "Is < 0");
    if (E > kMaxE) return fail(MOE_ERR_UNSUPPORTED, "E > 256");
    if (k > kMaxK) return fail(MOE_ERR_UNSUPPORTED, "k > 32");
    if (H % 64 != 0) return fail(MOE_ERR_UNSUPPORTED, "H is not a multiple of 64");
    if (need_I && I % 64 != 0) return fail(MOE_ERR_UNSUPPORTED, "I is not a multiple of 64");
    if (need_I && Is % 64 != 0) return fail(MOE_ERR_UNSUPPORTED, "Is is not a multiple of 64");
    if ((int64_t)T * (int64_t)k >= (int64_t(1) << 31)) return fail(MOE_ERR_UNSUPPORTED, "T * k >= 2^31");
    return Check{};
}

Check check_aligned(const void* p, const char* name, size_t align) {
    if (reinterpret_cast<uintptr_t>(p) % align != 0)
        return fail(MOE_ERR_MISALIGNED, std::string(name) + " is not " + std::to_string(align) + "-byte aligned");
    return Check{};
}

int router_splits(int T, int H, int E) {
    if (T <= kRouterSmallT) {
        // ~256 one-wave workgroups of 16 experts, but K ranges of at least 256 (a workgroup then reads 8 KB
        // or more of W_r; shorter ranges only multiply the partials the top-k kernel sums)
        const int64_t groups = (std::max(E, 1) + 15) / 16;
        int64_t s = (256 + groups - 1) / groups;
        s = std::max<int64_t>(1, std::min<int64_t>(s, std::min(kRouterMaxSplits, H / 256)));
        return (int)s;
    }
    // enough K ranges that the logits GEMM has >= 256 workgroups of 128 tokens, at most 32 and at most one
    // per 64-wide K chunk
    const int64_t tiles = ((int64_t)T + kWideBM - 1) / kWideBM;
    int64_t s = (256 + tiles - 1) / std::max<int64_t>(tiles, 1);
    s = std::max<int64_t>(1, std::min<int64_t>(s, std::min(32, H / 64)));
    return (int)s;
}

GemmPath gemm_path(int, int, int) { return GemmPath::Dma; }

int expected_active(int T, int E, int k) {
    if (T <= 0 || E <= 0 || k <= 0) return 0;
    const double miss = std::pow(1.0 - 1.0 / E, (double)T * k);
    return std::min(E, (int)std::ceil(E * (1.0 - miss) - 1e-9));
}

GemmPath dense_path(int) { return GemmPath::Dma; }

GemmPath fallback_path(int T, int E, int k) {
    const int64_t slots = (int64_t)T * k;
    if (slots <= (int64_t)kSkinnyBM * E) return GemmPath::Skinny;
    return slots < (int64_t)192 * E ? GemmPath::Wide : GemmPath::Tall;
}

int64_t max_tiles(int T, int E, int k, int BM) {
    const int64_t slots = (int64_t)T * k;
    return (slots + BM - 1) / BM + std::min<int64_t>(E, slots);
}

Layout forward_layout(int T, int H, int E, int k, int I, int Is, bool with_norm) {
    Layout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align_up(off + std::max<size_t>(bytes, 1), 256);
        return at;
    };
    const size_t Tk = (size_t)T * (size_t)k;
    const size_t chunks = ((size_t)T + kPermChunk - 1) / kPermChunk;
    L.ids = take(Tk * 4);
    L.gates = take(Tk * 4);
    L.counts = take((size_t)E * 4);
    L.offsets = take(((size_t)E + 1) * 4);
    L.row_token = take(Tk * 4);
    L.slot_row = take(Tk * 4);
    L.chunk_base = take(chunks * (size_t)E * 4);
    // room for the longest tile list any grouped-GEMM kernel can ask for (the smallest BM), with the
    // shared expert's tiles when it is folded in
    const int bm_min = std::min(std::min(kWideBM, kTallBM), kSkinnyBM);
    const bool fold = shared_fold(T, E, k, I, Is);
    L.tiles = take((size_t)(max_tiles(T, E, k, bm_min) + (fold ? shared_tiles(T, bm_min) : 0)) * kTileEntryBytes);
    L.ntiles = take(4);
    L.xcd_bounds = take((2 * (kXcds + 1) + 4 * kXcds) * 4); // two XCD splits, then 2 x kXcds 64-bit counters
    L.partial = take((size_t)router_splits(T, H, E) * (size_t)T * (size_t)E * 4);
    const size_t rows = Tk + (fold ? (size_t)T : 0);
    // h: the routed rows, then (shared expert of the routed width) its T rows, whether it runs as a group of
    // the routed GEMMs or as a dense MLP
    const bool same_width = Is > 0 && Is == I;
    L.h_perm = take((Tk + (same_width ? (size_t)T : 0)) * (size_t)I * 2);
    // per-slot rows: bf16 where slot_rows_bf16 holds (never with the shared expert folded in at decode), else
    // fp32; the decode fold's shared rows follow them
    L.y_perm = take(rows * (size_t)H * (slot_rows_bf16(T, E, k, I, Is) ? 2 : 4));
    const bool dense_shared = Is > 0 && !fold;
    L.h_sh = dense_shared && !same_width ? take((size_t)T * (size_t)Is * 2) : size_t(-1);
    L.y_sh = dense_shared ? take((size_t)T * (size_t)H * 4) : size_t(-1);
    const size_t shp = dense_shared ? dense_partial_bytes(T, H, Is) : 0;
    L.sh_partial = shp > 0 ? take(shp) : size_t(-1);
    const bool ks = ksplit_possible(T, H, E, k, I, Is);
    L.ks_flag = ks ? take(16) : size_t(-1); // the two GEMMs' splits, then their stream-K flags
    L.ks_part = ks ? take((size_t)kMaxGateUpSplits * rows * (size_t)I * 2 * 4) : size_t(-1);
    L.ks_part_down = ks ? take((size_t)(down_split_max(T) - 1) * rows * (size_t)H * 4) : size_t(-1);
    L.x_norm = with_norm ? take((size_t)T * (size_t)H * 2) : size_t(-1); // last: the block layout extends the plain one
    L.total = off;
    return L;
}

Check check_dense_sizes(int T, int H, int Id) {
    if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T < 0");
    if (H <= 0) return fail(MOE_ERR_INVALID_ARG, "H <= 0");
    if (Id <= 0) return fail(MOE_ERR_INVALID_ARG, "I <= 0");
    if (H % 64 != 0) return fail(MOE_ERR_UNSUPPORTED, "H is not a multiple of 64");
    if (Id % 64 != 0) return fail(MOE_ERR_UNSUPPORTED, "I is not a multiple of 64");
    if ((int64_t)T >= (int64_t(1) << 31) / 16) return fail(MOE_ERR_UNSUPPORTED, "T >= 2^27");
    return Check{};
}

int dense_splits(bool gate_up, int rows, int N, int K) {
    if (rows <= 0 || N <= 0 || K <= 0) return 1;
    const int64_t tiles = ((int64_t)rows + kSkinnyBM - 1) / kSkinnyBM;
    const int64_t ntn = gate_up ? N / 64 : (N + 127) / 128;
    const int64_t blocks = std::max<int64_t>(1, tiles * ntn);
    const int64_t want = (1024 + blocks - 1) / blocks;
    const int64_t cap = std::max<int64_t>(1, std::min<int64_t>(kMaxDenseSplits, K / 256));
    return (int)std::max<int64_t>(1, std::min(want, cap));
}

int dma_dense_splits(bool gate_up, int rows, int N, int K, int cus) {
    if (rows <= 0 || rows > kDmaSplitMaxT || N <= 0 || K <= 0 || cus <= 0) return 1;
    const int64_t tiles = ((int64_t)rows + kTallBM - 1) / kTallBM;
    const int64_t B = tiles * dma_ntn(gate_up, N);
    const int steps = K / 64;
    const int cap = std::max(1, std::min(kMaxDenseSplits, steps / 4));
    int best = 1;
    double best_t = 0;
    for (int S = 1; S <= cap; ++S) {
        const double t = (double)((B * S + cus - 1) / cus) * ((double)steps / S + 3.0);
        if (S == 1 || t < best_t) best = S, best_t = t;
    }
    return best;
}

int dma_stream_splits(bool gate_up, int rows, int N, int K, int cus) {
    const int steps = K / 64;
    if (rows <= 0 || N <= 0 || K <= 0 || cus <= 0 || steps % 4 != 0) return 0;
    if (rows > kDmaSplitMaxT) return 1;
    const int64_t B = (((int64_t)rows + kTallBM - 1) / kTallBM) * dma_ntn(gate_up, N);
    // One round of blocks that fills at least three quarters of the CUs first: fewer, longer ranges read
    // longer runs of each weight row, which streams faster than more rounds of shorter ones (GLM-5 dense MLP at
    // 16 tokens, down GEMM in 8 ranges: gate/up in 2 ranges, 192 blocks, 0.0928 ms; in 8, 768 blocks, 0.0981
    // ms; in 3, 288 blocks and a second round for 32 CUs, 0.121 ms).
    for (int S = 1; S <= kMaxDenseSplits && S <= steps / 4; ++S)
        if ((steps / 4) % S == 0 && 4 * B * S >= 3 * (int64_t)cus && B * S <= cus) return S;
    const double part_step = (double)rows * (gate_up ? 2 * N : N) * 8.0 / (32768.0 * cus);
    int best = 1;
    double best_t = 0;
    for (int S = 1; S <= kMaxDenseSplits && S <= steps / 4; ++S) {
        if ((steps / 4) % S != 0) continue;
        double t = (double)((B * S + cus - 1) / cus) * (double)(steps / S);
        if (S > 1) t += S * part_step + 2.0;
        if (S == 1 || t < best_t) best = S, best_t = t;
    }
    return best;
}

size_t dense_partial_bytes(int T, int H, int Id) {
    const int s1 = dense_splits(true, T, Id, H), s2 = dense_splits(false, T, H, Id);
    size_t a = s1 > 1 ? (size_t)s1 * T * 2 * Id * 4 : 0;
    size_t b = s2 > 1 ? (size_t)s2 * T * H * 4 : 0;
    if (T > 0 && T <= kDmaSplitMaxT) { // the LDS-copy kernel's splits, whatever the device's CU count
        const int m1 = std::max(1, std::min(kMaxDenseSplits, H / 256)), m2 = std::max(1, std::min(kMaxDenseSplits, Id / 256));
        if (m1 > 1) a = std::max(a, (size_t)m1 * T * 2 * Id * 4);
        if (m2 > 1) b = std::max(b, (size_t)m2 * T * H * 4);
    }
    return std::max(a, b);
}

size_t dense_workspace_bytes(int T, int H, int Id) {
    const size_t hb = align_up(std::max<size_t>((size_t)T * (size_t)Id * 2, 1), 256);
    return hb + align_up(dense_partial_bytes(T, H, Id), 256);
}

namespace {
// Workspace sizes are not monotone in T: regions appear and vanish with the regimes (the shared-expert fold,
// the decode K split, the dense shared expert), and the router's and the dense GEMMs' K splits step down as
// T grows. Between consecutive candidates below every region grows with T, so the largest size over
// T' <= T is the largest over T and the candidates: the multiples of 16 (the 16- and 128-row tile
// boundaries where the splits step down; past 32768 rows no split is left) and the last T of the fold and
// K-split regimes.
template <typename F>
size_t max_over_smaller(int T, int fold_end, F size_at) {
    size_t best = size_at(T);
    const int lim = std::min(T - 1, 32768);
    for (int t = 16; t <= lim; t += 16) best = std::max(best, size_at(t));
    for (int t : {fold_end, std::min(fold_end, kKSplitMaxT)})
        if (t >= 0 && t < T) best = std::max(best, size_at(t));
    return best;
}
} // namespace

size_t forward_workspace_bound(int T, int H, int E, int k, int I, int Is, bool with_norm) {
    // last T with the shared expert folded in (T * k <= kSkinnyBM * E), when it can fold at all
    const int fold_end = Is > 0 && Is == I ? (int)std::min<int64_t>((int64_t)kSkinnyBM * E / k, INT32_MAX) : -1;
    return max_over_smaller(T, fold_end,
                            [&](int t) { return forward_layout(t, H, E, k, I, Is, with_norm).total; });
}

size_t dense_workspace_bound(int T, int H, int Id) {
    return max_over_smaller(T, -1, [&](int t) { return dense_workspace_bytes(t, H, Id); });
}

size_t permute_scratch_bytes(int T, int E) {
    const size_t chunks = ((size_t)T + kPermChunk - 1) / kPermChunk;
    return align_up(std::max<size_t>(chunks * (size_t)E * 4, 1), 256);
}

} // namespace moe
