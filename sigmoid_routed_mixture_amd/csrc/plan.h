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
// one-wave workgroups of 16 experts x 32-wide K chunks, split so the launch has up to 256 workgroups with K
// ranges of at least 256 (at most kRouterMaxSplits ranges); above, on the wide GEMM kernel with 64-wide chunks
// (at most 32 ranges).
constexpr int kRouterSmallT = 16;
constexpr int kRouterMaxSplits = 64;
int router_splits(int T, int H, int E);
// Grouped GEMMs take the Dma kernel at every size (measured faster than the weight-streaming kernel from
// one token to 512 at the GLM-5 and GLM-4.7-Flash shapes, decode included).
GemmPath gemm_path(int T, int E, int k);
// A dense GEMM of T rows (shared expert, dense MLP): the Dma kernel, with split K up to kDmaSplitMaxT rows
// (one token tile cannot fill the GPU otherwise; measured faster than the weight-streaming kernel's split).
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
// Chunk-major order: the tile list is a sequence of chunks, each a run of consecutive tiles of one group
// (expert); the blocks of a chunk whose tiles are [first, first + cm) of the list are positions
// [first * ntn, (first + cm) * ntn) of the order, output-column tile 0 of every tile of the chunk first, then
// column tile 1, and so on (the chunk's tiles share each weight slice side by side). Position L lies in the
// chunk of the tile at L / ntn, which is tile ci of its chunk. Returns the block's tile-list index, sets its
// column tile.
constexpr int64_t chunk_major_tile(int64_t L, int ntn, int ci, int cm, int& ntile) {
    const int64_t first = L / ntn - ci;
    const int64_t r = L - first * ntn;
    ntile = (int)(r / cm);
    return first + r % cm;
}

// A tile of the device-side list is an int4 {word, first row of the tile in its group, rows of the group,
// first permuted row of the group}; the word packs the group (9 bits), the tile height (9 bits), the
// tile's index in its chunk (7 bits) and the chunk's tile count minus one (7 bits).
constexpr int kTileEntryBytes = 16;
constexpr int kMaxChunkTiles = 128;
constexpr int tile_word(int g, int ht, int ci, int cm) {
    return (int)((uint32_t)g | (uint32_t)ht << 9 | (uint32_t)ci << 18 | (uint32_t)(cm - 1) << 25);
}
constexpr int tile_group(int w) { return (int)((uint32_t)w & 511u); }
constexpr int tile_ht(int w) { return (int)(((uint32_t)w >> 9) & 511u); }
constexpr int tile_ci(int w) { return (int)(((uint32_t)w >> 18) & 127u); }
constexpr int tile_cm(int w) { return (int)(((uint32_t)w >> 25) & 127u) + 1; }
// Chunks of a group of nt tiles, chunk c of nc holding tiles [c nt / nc, (c + 1) nt / nc): in the plain order
// one chunk per kMaxChunkTiles tiles; in the dealt order (below) one per 4 tiles up to one per XCD (a big group
// spreads over every XCD, and each chunk's tiles share its weight slices), beyond 1024 tiles one per
// kMaxChunkTiles.
constexpr int plain_chunks(int nt, int cap = kMaxChunkTiles) { return nt <= 0 ? 0 : (nt + cap - 1) / cap; }
// Tiles per chunk of the plain order by default. A chunk's blocks run side by side on one XCD, its tiles
// sharing each weight slice and its column tiles each token tile; past ~16 tiles the blocks that share a
// token tile run too far apart to find it in L2 (a 32768-row expert in one chunk re-read its tokens from
// HBM for every column tile: the skewed GLM-5 workload 20.0 ms against 18.2 ms with chunks of 16).
constexpr int kPlainChunkTiles = 16;
constexpr int dealt_chunks(int nt) {
    if (nt <= 0) return 0;
    if (nt > kXcds * kMaxChunkTiles) return (nt + kMaxChunkTiles - 1) / kMaxChunkTiles;
    const int nc = (nt + 3) / 4;
    return nc < kXcds ? nc : kXcds;
}
constexpr int chunk_first(int c, int nc, int nt) { return (int)((int64_t)c * nt / nc); }

// Dealt order of the persistent routed GEMMs (prefill): the chunks of every group, the largest groups first
// (rows descending, then index; a folded shared expert before all), are dealt to the XCDs in snake order
// (0, 1, ..., 7, 7, 6, ..., 0, 0, 1, ...); XCD x's blocks are its chunks in dealing order. Each XCD thus gets
// a like share of big and small experts, the blocks that run side by side on an XCD have like heights, and
// its last blocks are its smallest. Up to kMaxDealtChunks chunks (else the plain order).
// Three forms: groups by size (rows descending) or by index; within an XCD the dealing order, or (by size)
// its chunks alternately from the largest and the smallest end.
enum DealtOrder { kDealtSorted = 1, kDealtIndex = 2, kDealtAlternating = 3 };
constexpr int kMaxDealtChunks = 2048;
constexpr int kDealtSlots = kMaxDealtChunks / kXcds; // chunks per XCD at most
constexpr int deal_xcd(int c) {
    const int j = c % (2 * kXcds);
    return j < kXcds ? j : 2 * kXcds - 1 - j;
}
constexpr int deal_slot(int c) { return 2 * (c / (2 * kXcds)) + (c % (2 * kXcds) >= kXcds ? 1 : 0); }
// Chunks XCD x receives when `total` chunks are dealt.
constexpr int deal_count(int x, int total) {
    const int q = total / (2 * kXcds), r = total % (2 * kXcds);
    return 2 * q + (x < r ? 1 : 0) + (2 * kXcds - 1 - x < r ? 1 : 0);
}
// Alternating form: slot s of the m slots of an XCD moves to place 2 s (its larger half) or 2 (m - 1 - s) + 1.
constexpr int alternate_slot(int s, int m) { return 2 * s < m ? 2 * s : 2 * (m - 1 - s) + 1; }

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
// Above the decode fold, the shared expert with the routed width can still be one more group of the
// persistent routed GEMMs (when the caller gives it no stream of its own): its tiles, cut into one chunk per
// XCD, are spread through the block order so that every XCD's range holds one; its h rows follow the T * k
// routed rows, its output goes to fp32 y_shared rows of its own (the routed per-slot rows may be bf16).
constexpr bool shared_fold_prefill(int T, int E, int k, int I, int Is) {
    return Is > 0 && Is == I && !shared_fold(T, E, k, I, Is);
}
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
// Experts a decode batch of T tokens is expected to reach with k picks each among E (uniform routing:
// E (1 - (1 - 1/E)^(T k))), rounded up. The gate/up GEMM gets room for a K split (and its reduction launch)
// only when decode_ksplit of that many experts' blocks (plus the folded shared expert's) would split.
int expected_active(int T, int E, int k);
// The down GEMM may cut K into more ranges at the smallest batches: up to kMaxDownSplits up to
// kDownSplit4MaxT tokens, 2 above (ranges 2 .. S write fp32 rows of their own, (S - 1) x rows x H x 4 bytes
// of workspace, which the combine adds in range order).
constexpr int kMaxDownSplits = 4;
constexpr int kDownSplit4MaxT = 16;
constexpr int down_split_max(int T) { return T <= kDownSplit4MaxT ? kMaxDownSplits : 2; }
// The gate/up GEMM's split: 1 or 2. From two rounds on, two half-length blocks per block pay when they round
// better, counting about 5 % for the extra prologues and the partials: 0.525 r2 < r1 (r_S the rounds of S b
// blocks on cus CUs).
constexpr int decode_ksplit(int64_t blocks, int cus) {
    if (blocks <= 0 || cus <= 0) return 1;
    const int64_t r1 = (blocks + cus - 1) / cus, r2 = (2 * blocks + cus - 1) / cus;
    return r1 >= 2 && 21 * r2 < 40 * r1 ? 2 : 1;
}
// The down GEMM's split among `allow` (bit S set for each allowed S, 2 <= S <= kMaxDownSplits): the fewest
// rounds per unit of work, r_S / S, with each range beyond two counted 5 % dearer (r_S (18 + S) / (20 S));
// two ranges are taken already when they round as well as one (its second range costs no launch: the
// combine adds it; GLM-5 decode, 1968 blocks: 1.0735 ms whole, 1.0678 ms in two, 1.1083 ms in four). One
// round already: no split.
constexpr int decode_ksplit_down(int64_t blocks, int cus, int allow) {
    if (blocks <= 0 || cus <= 0) return 1;
    const int64_t r1 = (blocks + cus - 1) / cus;
    if (r1 < 2) return 1;
    int best = 1;
    int64_t num = r1, den = 1; // cost of the best split so far, num / den
    for (int S = 2; S <= kMaxDownSplits; ++S) {
        if (!((allow >> S) & 1)) continue;
        const int64_t r = (S * blocks + cus - 1) / cus;
        const int64_t n = r * (18 + S), d = 20 * (int64_t)S; // r (18 + S) / (20 S)
        if (S == 2 ? n * den <= num * d : n * den < num * d) best = S, num = n, den = d;
    }
    return best;
}
// The gate/up GEMM's split among 1, 2 and (allow4: four ranges are whole ring periods) 4: decode_ksplit's
// choice, or 4 when two already pay, the half-length blocks take at least 8 rounds (the extra ranges' starts
// amortised) and quarter-length ones round strictly better (r4 < 2 r2). GLM-5 decode, 1296 blocks (11 rounds
// of halves, 21 of quarters): 1.0665 ms in two, 1.0621 ms in four (interleaved in one process).
constexpr int kMaxGateUpSplits = 4;
constexpr int decode_ksplit_gate_up(int64_t blocks, int cus, bool allow4) {
    const int S = decode_ksplit(blocks, cus);
    if (S != 2 || !allow4) return S;
    const int64_t r2 = (2 * blocks + cus - 1) / cus, r4 = (4 * blocks + cus - 1) / cus;
    return r2 >= 8 && r4 < 2 * r2 ? 4 : 2;
}
// Stream-K at decode: a streamed launch (below) of b live blocks, b at least the number of CUs (so every
// workgroup's share of the blocks' K steps is at least one block long and each block is cut at most once),
// gives each workgroup one contiguous share of the ring periods of all blocks: every CU streams the same
// number of weight bytes, where whole blocks or even splits leave the last round part-empty (GLM-4.7-Flash
// decode: 444 gate/up blocks, 1.73 rounds; 296 down blocks in three ranges, 3.47). The cut blocks write two
// fp32 planes that the gate/up reduction and the combine add, as for the split in two.
constexpr bool decode_streamk(int64_t blocks, int cus) { return cus > 0 && blocks >= cus; }
// A decode-sized grouped GEMM runs streamed (one workgroup per CU, its blocks back to back, the next block's
// first copies in flight during the current one's last steps) when the blocks it is expected to have, with
// the K split decode_ksplit would choose, come to at most 4 per CU: there the blocks' empty-ring starts
// weigh most (GLM-4.7-Flash decode, about 2 per CU: 2.8 % faster). With many blocks per CU the one-workgroup-
// per-block launch balances the tail better than the streamed form's fixed share (GLM-5 decode, 8-13 per
// CU: 1.1 % slower streamed).
constexpr bool decode_streamed(int64_t blocks, int cus) {
    return blocks > 0 && cus > 0 && blocks * decode_ksplit(blocks, cus) <= 4 * (int64_t)cus;
}


struct Layout {
    // byte offsets inside the workspace (each 256-byte aligned); size_t(-1) = not present
    size_t ids, gates, counts, offsets, row_token, slot_row, chunk_base, tiles, ntiles, xcd_bounds, partial,
        h_perm, y_perm, h_sh, y_sh, sh_partial, x_norm, ks_flag, ks_part, ks_part_down;
    size_t total;
};
// with_norm adds a [T, H] bf16 region for the RMS-normalised stream of the block entry point.
// ks_flag / ks_part / ks_part_down: the device's K-split choices (gate/up, down: two ints, then their two
// stream-K flags), the gate/up
// partials [2][T·k + T][2I] fp32 and the rows of the down GEMM's ranges 2 .. S, [down_split_max(T) - 1]
// [T·k + T][H] fp32, of a decode-sized launch (ksplit_possible), else not present.
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
// A dense GEMM of up to kDmaSplitMaxT rows on the LDS-copy kernel has too few blocks (one token tile times
// the column tiles) to fill the GPU, so it splits K into S ranges of at least 4 K steps (S <= kMaxDenseSplits):
// the S that minimises the launch's rounds of blocks, ceil(B S / cus), times a block's length in K steps plus
// 3 steps of prologue, (K / 64) / S + 3 (B blocks unsplit). The ranges write fp32 partials, which a reduction
// kernel adds in K order.
constexpr int kDmaSplitMaxT = 64;
// Up to this many tokens every tile of a launch has at most 32 rows (a group never holds more rows than there
// are tokens), and the LDS-copy kernel runs with its deeper copy ring.
constexpr int kDeepRingMaxT = 32;
int dma_dense_splits(bool gate_up, int rows, int N, int K, int cus);
// The same choice for the streamed form of that kernel (one workgroup per CU running its blocks back to back,
// the next block's first copies in flight during the last steps of the one before): ranges of equal length, a
// multiple of 4 K steps (the copy ring's period), so S divides (K / 64) / 4. The smallest S whose B S blocks
// make one round filling at least three quarters of the CUs; failing that, the S that minimises the rounds of
// blocks times a block's length, ceil(B S / cus) * (K / 64) / S, plus, when S > 1, the partials' round trip
// ((S rows N' 8) bytes in steps of cus * 32 KB, N' = 2N for gate/up, N for down) and 2 steps for the reduction
// launch. 0 when K / 64 is not a multiple of 4 (the kernel's one-workgroup-per-block form runs).
int dma_stream_splits(bool gate_up, int rows, int N, int K, int cus);
// fp32 partials of a dense SwiGLU MLP (gate/up then down, one region reused) on that kernel; 0 if unsplit.
size_t dense_partial_bytes(int T, int H, int Id);

// Dense SwiGLU MLP: T >= 0, H and Id positive multiples of 64. Its workspace is h [T, Id] bf16 and the
// split partials.
Check check_dense_sizes(int T, int H, int Id);
size_t dense_workspace_bytes(int T, int H, int Id);
// The largest dense_workspace_bytes(T', H, Id) over T' <= T.
size_t dense_workspace_bound(int T, int H, int Id);

} // namespace moe
