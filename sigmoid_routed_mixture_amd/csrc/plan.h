// Host-side argument checks, launch planning and workspace layout of the MoE layer.
// Pure C++: no HIP types or calls, so every rule here runs (and is tested) without a GPU.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

#include "moe.h"

namespace moe {

// Tile shapes the kernels are built for (the kernels static_assert against these).
constexpr int kWideBM = 128;    // tokens per tile of the LDS-tiled grouped GEMM
constexpr int kTallBM = 256;    // tokens per tile of its tall variant (experts of >= 192 rows on average)
constexpr int kSkinnyBM = 16;   // tokens per tile of the weight-streaming grouped GEMM
constexpr int kRouterBT = 32;   // tokens per router workgroup
constexpr int kPermChunk = 256; // tokens per permutation chunk
constexpr int kMaxE = 256;
constexpr int kMaxK = 32;
constexpr int kMaxDenseSplits = 16; // K ranges of a dense GEMM on the weight-streaming kernel

// Grouped-GEMM kernels: Dma (256-token tiles, both operands loaded straight into LDS), Wide and Tall (128-
// and 256-token tiles, weights streamed through registers: the fallback when an operand is too large for
// Dma's 32-bit offsets, and Wide for the router logits), Skinny (16-token tiles, decode).
enum class GemmPath { Wide, Tall, Dma, Skinny };
constexpr int path_bm(GemmPath p) {
    return p == GemmPath::Tall || p == GemmPath::Dma ? kTallBM : p == GemmPath::Wide ? kWideBM : kSkinnyBM;
}
// The Dma kernel addresses each operand as a 32-bit byte offset from a base: a matrix of `rows` rows of K
// bf16 must stay below 4 GiB.
constexpr bool dma_fits(int64_t rows, int64_t K) { return rows * K * 2 < (int64_t(1) << 32); }

struct Check {
    moe_status status = MOE_OK;
    std::string message;
    bool ok() const { return status == MOE_OK; }
};

// Size rules shared by every entry point. I and Is are ignored when negative-one (router/permute).
Check check_sizes(int T, int H, int E, int k, int I, int Is, bool need_I);
Check check_aligned(const void* p, const char* name, size_t align = 16);

// K-split of the router's logit GEMM: the number of K ranges. Up to kRouterSmallT tokens the logits run on
// one-wave workgroups of 16 experts x 32-wide K chunks, split so the launch has >= 256 workgroups (at most
// kRouterMaxSplits ranges); above, on the wide GEMM kernel with 64-wide chunks (at most 32 ranges).
constexpr int kRouterSmallT = 16;
constexpr int kRouterMaxSplits = 64;
int router_splits(int T, int H, int E);
// Grouped GEMMs take the Dma kernel at every size (measured faster than the weight-streaming kernel from
// one token to 512 at the GLM-5 and GLM-4.7-Flash shapes, decode included).
GemmPath gemm_path(int T, int E, int k);
// A dense GEMM of T rows (shared expert, dense MLP): the weight-streaming kernel with split K up to 16 rows
// (one token tile cannot fill the GPU otherwise), else the Dma kernel.
GemmPath dense_path(int T);
// When an operand does not fit the Dma kernel: the weight-streaming kernel when experts average at most 16
// rows, else the register-streaming one with 128-token tiles below 192 rows on average and 256-token
// tiles from there.
GemmPath fallback_path(int T, int E, int k);
// Upper bound of grouped-GEMM tiles of BM rows over all experts: sum_e ceil(n_e / BM).
int64_t max_tiles(int T, int E, int k, int BM);

// Height of the tiles an expert with n rows is cut into (the last tile may be shorter). For the LDS-tiled
// kernel the rows are split evenly over ceil(n / BM) tiles, rounded up to 16 rows (BM 128) or 32 rows
// (BM 256, whose kernel is compiled for even block counts): an expert's tiles then compute about the same
// number of 16-row blocks, run in step and share its weights in L2. The 16-row kernel cuts at BM. The tile
// count is ceil(n / height) <= ceil(n / BM).
constexpr int tile_height(int n, int BM) {
    if ((BM != kTallBM && BM != kWideBM) || n <= 0) return BM;
    const int q = BM == kTallBM ? 32 : 16;
    const int nt = (n + BM - 1) / BM;
    const int h = ((n + nt - 1) / nt + q - 1) / q * q;
    return h < BM ? h : BM;
}

// Workgroup order of the LDS-tiled grouped GEMM (pure arithmetic, also used by the kernel).
// The hardware hands workgroup b to XCD b % kXcds and each XCD has its own L2, so the `live` blocks are
// put in one order and XCD x takes the x-th contiguous chunk of it. Returns the block's position L in
// that order, or -1 when workgroup `bid` has no block (the grid is padded to a multiple of kXcds).
constexpr int kXcds = 8;
constexpr int64_t xcd_block_order(int64_t bid, int64_t live) {
    const int64_t chunk = (live + kXcds - 1) / kXcds;
    const int64_t local = bid / kXcds;
    const int64_t L = (bid % kXcds) * chunk + local;
    return (local < chunk && L < live) ? L : -1;
}
// Expert-major order: position L lies in the range of an expert whose tiles are [first, first + m) of
// the tile list (L / ntn is tile i of the expert); inside the range, output-column tile 0 of every token
// tile comes first, then column tile 1, and so on. Returns the tile-list index, sets the column tile.
constexpr int64_t expert_major_tile(int64_t L, int ntn, int i, int m, int& ntile) {
    const int64_t first = L / ntn - i;
    const int64_t r = L - first * ntn;
    ntile = (int)(r / m);
    return first + r % m;
}

// Work-balanced split of the DMA kernel's grouped blocks over the XCDs: XCD x takes blocks
// [bounds[x], bounds[x + 1]) of the expert-major order, at most dma_xcd_cap(...) of them (the grid gives
// each XCD that many workgroups). A block's work is counted as its 32-row token blocks plus
// kDmaBlockCost for the weight slice every block streams.
constexpr int kDmaBlockCost = 2;
constexpr int dma_ntn(bool gate_up, int N) { return gate_up ? (N + 127) / 128 : (N + 255) / 256; }
constexpr int64_t dma_xcd_cap(int64_t grid_tiles, int ntn) {
    const int64_t avg = (grid_tiles * ntn + kXcds - 1) / kXcds;
    return avg + avg / 4 + 1;
}

// Block claims of the persistent DMA kernel. An XCD's range [lo, hi) is handed out through one 64-bit counter:
// the home XCD's workgroups add kClaimFront and take the range from the front, workgroups of other XCDs add
// kClaimBack and take it from the back. Every claim raises front + back by one, so the claims that saw
// front + back < hi - lo get distinct blocks and all later ones get none. `old` is what the atomic add
// returned; the result is the claimed block or -1.
constexpr uint64_t kClaimFront = 1, kClaimBack = uint64_t(1) << 32;
constexpr int64_t claim_block(int lo, int hi, uint64_t old, bool home) {
    const int64_t f = (int64_t)(old & 0xFFFFFFFFu), b = (int64_t)(old >> 32);
    return f + b < (int64_t)hi - lo ? (home ? lo + f : hi - 1 - b) : -1;
}

// With few tokens per expert (at most 16 on average) the shared expert joins the routed experts' grouped
// GEMMs as one more group (index E, all T tokens, its rows after the T * k routed rows) when it has the
// routed experts' width: its weights then stream with theirs in one launch. Otherwise it runs as two dense
// GEMMs of its own (with many tokens the dense tile order reuses its weights better than one more group).
constexpr bool shared_fold(int T, int E, int k, int I, int Is) {
    return Is > 0 && Is == I && (int64_t)T * k <= (int64_t)kSkinnyBM * E;
}
constexpr int64_t shared_tiles(int T, int BM) { return ((int64_t)T + BM - 1) / BM; }
// The down GEMM's per-slot rows (read back once by the combine) are stored as bf16 when every token has at
// least 8 gated slots and the shared expert is not folded in (so neither a K split nor shared rows are among
// them), else as fp32. A bf16 row adds one rounding of each slot's output before the fp32 weighted sum; over
// 8 or more slots these roundings partly cancel (simulated worst case about 0.010 x the output RMS at k = 8,
// 0.013-0.015 at k = 4 and up to 0.020 at k = 1, where h's own bf16 rounding alone gives 0.008-0.012).
constexpr bool slot_rows_bf16(int T, int E, int k, int I, int Is) { return k >= 8 && !shared_fold(T, E, k, I, Is); }
// Decode-sized grouped GEMMs (the shared expert folded in, at most kKSplitMaxT tokens, K of at least two
// steps) may split K in two. Every CU runs one DMA block at a time, so a launch of b blocks takes
// ceil(b / cus) rounds; from two rounds on, two half-length blocks per block pay when they round better,
// counting about 5 % for the extra prologues and the fp32 partials (in one round the fixed costs win). The permutation picks the split from the live block
// count, so the GEMM and the reduction that follows agree on it.
constexpr int kKSplitMaxT = 64;
constexpr int decode_ksplit(int64_t blocks, int cus) {
    if (blocks <= 0 || cus <= 0) return 1;
    const int64_t r1 = (blocks + cus - 1) / cus, r2 = (2 * blocks + cus - 1) / cus;
    return r1 >= 2 && 21 * r2 < 40 * r1 ? 2 : 1; // one round already: no split; else 0.525 r2 < r1
}

// A tile of the device-side list: {group | tile height << 16, first row in the group, rows of the group,
// first permuted row of the group} (int4), so a workgroup decodes its block with one load.
constexpr int kTileEntryBytes = 16;

struct Layout {
    // byte offsets inside the workspace (each 256-byte aligned); size_t(-1) = not present
    size_t ids, gates, counts, offsets, row_token, slot_row, chunk_base, tiles, ntiles, xcd_bounds, partial,
        h_perm, y_perm, h_sh, y_sh, sh_partial, x_norm, ks_flag, ks_part, ks_part_down;
    size_t total;
};
// with_norm adds a [T, H] bf16 region for the RMS-normalised stream of the block entry point.
// ks_flag / ks_part / ks_part_down: the device's K-split choices (gate/up, down: two ints), the gate/up
// partials [2][T·k + T][2I] fp32 and the down GEMM's second-half rows [T·k + T][H] fp32 of a decode-sized
// launch (ksplit_possible), else not present.
Layout forward_layout(int T, int H, int E, int k, int I, int Is, bool with_norm = false);
constexpr bool ksplit_possible(int T, int H, int E, int k, int I, int Is) {
    return shared_fold(T, E, k, I, Is) && T <= kKSplitMaxT && H >= 128 && I >= 128; // a K step per half
}
// What a caller allocates for up to T tokens: the largest forward_layout(T', ...).total over T' <= T (the
// layouts are not monotone in T), so one workspace sized for the largest batch serves every smaller one.
size_t forward_workspace_bound(int T, int H, int E, int k, int I, int Is, bool with_norm = false);
size_t permute_scratch_bytes(int T, int E);

// K ranges of a dense GEMM (rows x N outputs, reduction K) on the weight-streaming kernel: enough for
// ~1024 workgroups, at most kMaxDenseSplits, each range at least 256 wide. 1 = no split.
int dense_splits(bool gate_up, int rows, int N, int K);
// fp32 partials of a dense SwiGLU MLP (gate/up then down, one region reused) on that kernel; 0 if unsplit.
size_t dense_partial_bytes(int T, int H, int Id);

// Dense SwiGLU MLP: T >= 0, H and Id positive multiples of 64. Its workspace is h [T, Id] bf16 and the
// split partials.
Check check_dense_sizes(int T, int H, int Id);
size_t dense_workspace_bytes(int T, int H, int Id);
// The largest dense_workspace_bytes(T', H, Id) over T' <= T.
size_t dense_workspace_bound(int T, int H, int Id);

} // namespace moe
