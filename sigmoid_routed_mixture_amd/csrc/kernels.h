// Launchers of the gfx950 kernels (host side). Each enqueues on `stream` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace moe {

// Router: logits, sigmoid, biased top-k, gates. With `partial` ([S, T, E] fp32 scratch, S from
// router_splits) the logits run K-split into fp32 partials (up to 16 tokens: one-wave workgroups of 16
// experts; above: the wide GEMM kernel) and a top-k kernel sums the S partials in order; without it one
// fused kernel (32 tokens per workgroup) does everything.
hipError_t launch_router(const uint16_t* x, const uint16_t* wr, const float* bias, int T, int H, int E, int k,
                         float scale, int32_t* ids, float* gates, float* logits, float* partial, int S,
                         hipStream_t stream);

// The logits alone of up to kRouterSmallT tokens (router_small_kernel: fp32 partials [S, T, E]); with
// `ticket` its first workgroup also zeroes that int for launch_route_permute_few.
hipError_t launch_router_logits_small(const uint16_t* x, const uint16_t* wr, int T, int H, int E, float* partial,
                                     int S, int32_t* ticket, hipStream_t stream);

// Permutation: per-chunk expert histograms, the prefix sums (and, when `tiles` is non-null, the list of
// BM-row grouped-GEMM tiles, kTileEntryBytes each), then the stable scatter of slots into expert-contiguous
// rows.
// chunk_scratch holds ceil(T / 256) * E ints.
// With shared_rows > 0 the tile list ends with the folded shared expert's tiles (group E). With `bounds`
// (no folded shared expert) it also writes, for the two column-tile counts ntn[0] and ntn[1] of the DMA
// kernel's two GEMMs, the work-balanced XCD split of their blocks (kXcds + 1 ints each, every XCD taking
// at most cap[i] blocks). With `ctr` (8-byte aligned) it zeroes the 2 * kXcds 64-bit work counters of the
// persistent DMA kernel (kXcds for each GEMM).
// With `ksplit` it writes the K splits of the gate/up and down GEMMs (two ints: decode_ksplit_gate_up and
// decode_ksplit_down of the live blocks, ks_ntn[i] column tiles each, on `cus` compute units, among the splits
// ks_allow[i] allows; ks_force > 0 forces one), then two stream-K flags: 1 where ks_streamk[i] allows it,
// nothing is forced, the split in two is allowed and the GEMM has at least `cus` live blocks (its split is
// then 2: the streamed kernel cuts each block at most once, the other kernels in halves, into the same two
// planes).
// With `dealt` (and `bounds`) the tile list takes a dealt order of plan.h (DealtOrder) and `bounds` the exact
// XCD ranges of that order for both GEMMs (when the chunks fit kMaxDealtChunks; else the plain order and
// split). The plain order cuts groups into chunks of at most plain_cap tiles.
struct XcdSplit {
    int32_t* bounds;
    int ntn[2];
    int cap[2];
    int32_t* ctr;
    int32_t* ksplit;
    int ks_ntn[2];
    int ks_allow[2]; // splits each GEMM may take: bit S set for S allowed (1 always is)
    int cus;
    int ks_force;    // 0 by the rule, 2 split in two, 3 the largest allowed split
    int ks_streamk[2]; // the GEMM's launch is streamed and may take stream-K (the gate/up reduction is enqueued)
    int dealt;
    int plain_cap;
    int spread_shared; // plain order: the shared group's tiles in kXcds chunks spread through the list
};
hipError_t launch_permute(const int32_t* ids, int T, int E, int k, int32_t* counts, int32_t* offsets,
                          int32_t* row_token, int32_t* slot_row, int32_t* chunk_scratch, int4* tiles,
                          int32_t* ntiles, int BM, int shared_rows, const XcdSplit& split, hipStream_t stream);

// Top-k of up to kRouterSmallT tokens from the partials launch_router_logits_small wrote (summed in split
// order, as launch_router does), then the single-chunk permutation of launch_permute, in one launch: one
// workgroup per token; the last to finish (counted on `ticket`, which the logits launch zeroed) permutes
// every token's ids. Writes what launch_router and launch_permute write, bit for bit.
hipError_t launch_route_permute_few(const float* partial, int S, const float* bias, int T, int E, int k, float scale,
                                    int32_t* ids, float* gates, float* logits, int32_t* ticket, int32_t* counts,
                                    int32_t* offsets, int32_t* row_token, int32_t* slot_row, int4* tiles,
                                    int32_t* ntiles, int BM, int shared_rows, const XcdSplit& split,
                                    hipStream_t stream);

// x_perm[r] = x[row_token[r]] for r < offsets[E].
hipError_t launch_gather_rows(const uint16_t* x, const int32_t* row_token, const int32_t* offsets, int E, int T,
                              int H, int rows_max, uint16_t* x_perm, hipStream_t stream);

// One grouped GEMM over the tile list (or, with counts == nullptr, one dense group of dense_rows rows).
struct GemmArgs {
    const uint16_t* act;       // activations [*, K] bf16
    const int32_t* row_token;  // gather map row -> activation row (gate/up GEMM of routed experts), or null
    const uint16_t* w_a;       // weights [groups][N][K] (down: W2; gate/up: W1)
    const uint16_t* w_b;       // gate/up only: W3 [groups][N][K]
    void* out;                 // [rows, N]: bf16 (h; grouped down with out_bf16) or fp32
    const int32_t* counts;     // rows per group, or null for one dense group
    const int32_t* offsets;    // first row of each group
    const int4* tiles;         // per tile {tile_word (group, height, place in its chunk), first row in the
                               // group, rows of the group, first permuted row of the group} (plan.h)
    const int32_t* ntiles;     // number of valid tiles
    int dense_rows;            // rows of the dense group (also the row count of each logits split)
    int groups;                // number of groups (routed experts); tiles naming another group are skipped
    int N, K;                  // output width (gate/up: I, h columns), reduction length
    const uint16_t* ws_a;      // grouped: the folded shared expert's weights (group `groups`), [N][K]: Ws1 / Ws2
    const uint16_t* ws_b;      // gate/up: Ws3
    int shared_rows;           // grouped: tokens of the folded shared expert (0: none), taken in token order
    int shared_off;            // its first row in the permuted buffers (T * k)
    const int32_t* xcd_bounds; // DMA kernel, grouped: the XCD split of the blocks (kXcds + 1 ints), or null
    unsigned long long* work_ctr; // DMA kernel, grouped: kXcds counters, zero at launch, for the persistent
                                  // form (one workgroup per CU claiming blocks), or null for one block each
    int ksplit;                // logits, and dense weight-streaming GEMMs: K ranges, each writing its own fp32
                               // partial ([dense_rows, N]; gate/up: [dense_rows, 2N], g then u)
    const int32_t* ksplit_dev; // DMA kernel, grouped: the K split S the permutation chose, or null; [2] is
                               // the stream-K flag (the streamed kernel's cut of each block in two planes)
    int ks_allow;              // with ksplit_dev: the splits it may hold (bit S set; gate/up at most
                               // kMaxGateUpSplits, down at most kMaxDownSplits)
    float* part;               // with a split: gate/up fp32 partials [S][part_rows][2N] (g, then u); down: the
                               // fp32 rows of K ranges 2 .. S, [S - 1][part_rows][N] (range 1 goes to out)
    int part_rows;
    int out_bf16;              // grouped down GEMM: per-slot rows stored as bf16 (slot_rows_bf16), else fp32
    float* out_shared;         // grouped down GEMM (LDS-copy kernel): fp32 rows [shared_rows, N] of the folded
                               // shared expert, row = its token, or null (its rows then follow the routed ones)
    int deep;                  // LDS-copy kernel, not persistent: every tile has at most 32 rows, so the deeper
                               // copy ring (three K steps of weights ahead) runs: 1 one workgroup per block,
                               // 2 streamed (one workgroup per CU runs blocks back to back, the next block's
                               // first copies issued during the last steps of the one before) where the shape
                               // allows it, else as 1
    int rt_rows;               // streamed grouped gate/up: entries of row_token (T * k, at most 1024)
};
enum class GemmKind { GateUp, DownF32, Logits };
hipError_t launch_gemm(GemmKind kind, GemmPath path, const GemmArgs& a, int64_t grid_tiles, hipStream_t stream);

// In-order reduction of a split dense GEMM's partials (dense_splits in plan.h) into h (gate/up, bf16 after
// the SwiGLU) or the fp32 output (down).
hipError_t launch_reduce(GemmKind kind, const float* partial, int S, int rows, int N, void* out, hipStream_t stream);
// The same for a grouped gate/up launch whose K split the device chose (*ksplit): nothing when it is 1.
hipError_t launch_reduce_ksplit(const float* partial, const int32_t* ksplit, int rows, int N, uint16_t* h,
                                hipStream_t stream);
// Compute units of the current device.
hipError_t device_cus(int& cus);

// out[t] = sum_j gates[t, j] * y[slot_row[t, j]] (+ y_shared[t]) (+ resid[t]), fp32, slot order, the
// residual (bf16) added last. The rows of y are bf16 when y_bf16, else fp32; y_shared is fp32. With
// `ysplit` (a device int S > 1) the down GEMM split K into S ranges: each row of y and y_shared is its first
// range plus the same row of y2 + p * part_stride / y_shared2 + p * part_stride for p = 0 .. S - 2, added
// in that order (fp32 rows only).
hipError_t launch_combine(const void* y, bool y_bf16, const float* gates, const int32_t* slot_row,
                          const float* y_shared, const uint16_t* resid, int T, int H, int k, float* out,
                          hipStream_t stream, const float* y2 = nullptr, const float* y_shared2 = nullptr,
                          const int32_t* ysplit = nullptr, size_t part_stride = 0);

// out[t] = bf16(gamma * x[t] / sqrt(mean(x[t]^2) + eps)), computed in fp64.
hipError_t launch_rmsnorm(const uint16_t* x, const uint16_t* gamma, double eps, int T, int H, uint16_t* out,
                          hipStream_t stream);

// Fills n ints with v.
hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t stream);

} // namespace moe
