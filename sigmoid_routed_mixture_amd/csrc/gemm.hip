// Grouped GEMMs of the SwiGLU experts on gfx950 (bf16 MFMA 16x16x32, fp32 accumulation).
//
// Gate/up GEMM: for the rows of one expert, g = x W1^T and u = x W3^T for the same output columns in one
// workgroup, and the epilogue writes h = silu(g) * u as bf16. Down GEMM: y = h W2^T, written as fp32 rows
// (per slot for the routed experts). Pages: open-model-atlas GLM-5 "MoE transformer block",
// "All 43 steps": g = x W1, u = x W3, a = g sigma(g), h = a * u, E_i = h W2, and the same four steps for
// the shared expert.
//
// Weights are the MFMA A operand (rows = output features) and tokens the B operand (columns), so a lane's
// four accumulator elements are four consecutive output features of one token row: 8-byte bf16 stores.
//
// Three kernels:
//  * dma    : up to 256 tokens x 256 weight rows per 8-wave workgroup, both operands copied from global
//             memory straight into LDS (buffer loads to LDS), weights two K steps ahead, tokens one; the
//             prefill kernel. The routed GEMMs run it persistent: one workgroup per CU claims blocks from
//             per-XCD counters.
//  * wide   : 128 or 256 tokens x 256 weight rows per 8-wave workgroup. Each wave streams its own 32
//             weight rows from HBM into MFMA registers; the token tile goes through double-buffered LDS.
//             The router logits (dense, K split across workgroups), and the fallback for operands past
//             the dma kernel's 32-bit offsets.
//  * skinny : 16 tokens per tile for experts with few rows (decode). No LDS: each wave streams its own
//             weight rows straight from HBM with 32-byte loads per lane, two 64-wide K chunks in flight
//             ahead of its MFMAs, so the kernel runs at the weight-streaming bound.
// All take their (expert, first row) tiles from the device-side list the permutation builds; the grid is
// an upper bound and workgroups past the list's length exit at once.
#include <atomic>

#include "common.h"
#include "kernels.h"
#include "plan.h"

namespace moe {
namespace {

constexpr int kBK = 64;

// The K split the permutation chose for a decode-sized grouped launch (1 .. kMaxDownSplits).
__device__ __forceinline__ int device_split(const int32_t* ksplit) {
    const int S = ksplit[0];
    return S < 1 ? 1 : S > kMaxDownSplits ? kMaxDownSplits : S;
}

struct TileInfo {
    int g, m0, rows, off;
    bool shared; // the folded shared expert (group index == groups)
};

// Row n of a group's weights: routed experts from w ([groups][N][K]), the folded shared expert from ws.
__device__ __forceinline__ const uint16_t* weight_row(const uint16_t* w, const uint16_t* ws, const TileInfo& ti,
                                                      int N, int n, int K) {
    return ti.shared ? ws + (size_t)n * K : w + ((size_t)ti.g * N + n) * K;
}

// A tile of the list: {tile_word (group, tile height, place in its chunk), first row in the group, rows of
// the group, first permuted row of the group} (plan.h); the folded shared expert is group `groups`.
template <int BM>
__device__ __forceinline__ bool entry_ok(const GemmArgs& a, const int4& e) {
    const int g = tile_group(e.x), ht = tile_ht(e.x);
    const int ngroups = a.groups + (a.shared_rows > 0 ? 1 : 0);
    return g < ngroups && ht > 0 && ht <= BM && tile_ci(e.x) < tile_cm(e.x) && e.y >= 0 && e.y < e.z && e.w >= 0;
}

template <bool DENSE, int BM>
__device__ __forceinline__ bool tile_info(const GemmArgs& a, int64_t mtile, TileInfo& ti) {
    if (DENSE) {
        ti.g = 0;
        ti.m0 = (int)(mtile * BM);
        ti.off = 0;
        ti.rows = min(BM, a.dense_rows - ti.m0);
        ti.shared = false;
        return ti.rows > 0;
    }
    if (mtile >= a.ntiles[0]) return false;
    const int4 t = a.tiles[mtile];
    if (!entry_ok<BM>(a, t)) return false;
    ti.g = tile_group(t.x);
    ti.m0 = t.y;
    ti.shared = ti.g == a.groups;
    ti.off = t.w;
    ti.rows = min(tile_ht(t.x), t.z - t.y);
    return true;
}

// Workgroup -> (token tile, output-column tile) of the grouped GEMMs. The live blocks go in chunk-major
// order (plan.h) and each XCD takes one range of it: the token tiles of a chunk that share a slice of an
// expert's weights run side by side on one XCD, and so do the column tiles that share a token tile, so
// both come from HBM about once instead of once per XCD.
// Block L of the order, decoded from the one entry at L / ntn (a tile of the same chunk): the tiles of a
// chunk are consecutive tiles of one group, so the block's tile is known without reading its own entry.
// `e` is the entry at L / ntn.
template <int BM>
__device__ __forceinline__ bool block_from(const GemmArgs& a, int ntn, int64_t L, const int4& e, TileInfo& ti,
                                           int& ntile) {
    const int64_t at = L / ntn;
    if (!entry_ok<BM>(a, e)) return false;
    const int ht = tile_ht(e.x);
    const int64_t t = chunk_major_tile(L, ntn, tile_ci(e.x), tile_cm(e.x), ntile);
    ti.g = tile_group(e.x);
    ti.m0 = e.y + (int)(t - at) * ht;
    ti.shared = ti.g == a.groups;
    ti.off = e.w;
    ti.rows = min(ht, e.z - ti.m0);
    return ti.rows > 0;
}
template <int BM>
__device__ __forceinline__ bool block_at(const GemmArgs& a, int ntn, int64_t L, TileInfo& ti, int& ntile) {
    return block_from<BM>(a, ntn, L, a.tiles[L / ntn], ti, ntile);
}

// With a K split of S, S consecutive positions of the order are the K ranges of one block (`ks` is the range).
template <int BM>
__device__ __forceinline__ bool grouped_block(const GemmArgs& a, int ntn, int64_t bid, TileInfo& ti, int& ntile,
                                              int S = 1, int* ks = nullptr) {
    const int64_t L = xcd_block_order(bid, (int64_t)a.ntiles[0] * ntn * S);
    if (L < 0) return false;
    if (ks != nullptr) *ks = (int)(L % S);
    return block_at<BM>(a, ntn, L / S, ti, ntile);
}

// The same order with the work-balanced XCD split the permutation wrote: XCD x = bid % kXcds takes the
// blocks [bounds[x], bounds[x + 1]).
template <int BM>
__device__ __forceinline__ bool balanced_block(const GemmArgs& a, int ntn, int64_t bid, TileInfo& ti, int& ntile) {
    const int x = (int)(bid % kXcds);
    const int64_t L = a.xcd_bounds[x] + bid / kXcds;
    if (L >= a.xcd_bounds[x + 1]) return false;
    return block_at<BM>(a, ntn, L, ti, ntile);
}

// Activation row for tile row m (clamped to the tile's last valid row: padded columns of the MFMA tile
// read a real row and are never stored).
template <GemmKind KIND, bool DENSE>
__device__ __forceinline__ const uint16_t* act_row(const GemmArgs& a, const TileInfo& ti, int m) {
    m = m < ti.rows ? m : ti.rows - 1;
    const int r = ti.off + ti.m0 + m;
    if (KIND == GemmKind::GateUp && !DENSE)
        return a.act + (size_t)(ti.shared ? ti.m0 + m : a.row_token[r]) * a.K; // the shared group takes every token
    return a.act + (size_t)r * a.K;
}

// ------------------------------------------------------------------------------------------------
// wide kernel

constexpr int kWaves = 8;            // waves per workgroup (two per SIMD)
constexpr int kWaveRows = 32;        // weight rows per wave: 2 MFMA row blocks of 16
constexpr int kWBN = kWaves * kWaveRows;  // weight rows per workgroup
constexpr int kWThreads = 64 * kWaves;

// Tile heights: 128 tokens (8 MFMA column blocks) or 256 (16). The taller tile loads a third fewer bytes
// per FLOP through the L1, which bounds this kernel (each CU keeps about 64 cache-line misses in flight
// at ~450 cycles of L2 latency); it holds one K step of token loads in registers instead of two to stay
// within 256 registers, and reads token fragments in groups of four blocks.
template <int BM>
struct WideShape {
    static_assert(BM == kWideBM || BM == kTallBM, "wide tiling assumes 128 or 256 tokens");
    static constexpr int XQ = BM / 64;               // token-row loads per thread per K step
    static constexpr int XS = BM == kWideBM ? 2 : 1; // token register stages (loads XS steps ahead)
    static constexpr int G = BM == kWideBM ? 8 : 4;  // token blocks per fragment group
};

// LDS token tile: [BM rows][64 k] bf16 (128 B per row); 16-byte chunk c of row r lives at chunk
// c ^ (r & 7) ^ ((r >> 3) & 1). An MFMA fragment read is 16 lanes on rows r..r+15 (r a multiple of 16) at
// one chunk: the permutation gives every 8 consecutive rows distinct chunks, and even rows (and odd
// rows) distinct chunks, so the 16 lanes cover all 64 four-byte banks and each 8-lane half all 32 of a
// 128-byte line: no bank conflicts whether the LDS serves 8 or 16 lanes of a b128 read per cycle.
__device__ __forceinline__ int lds_off(int row, int chunk) {
    return row * kBK + ((chunk ^ (row & 7) ^ ((row >> 3) & 1)) << 3);
}

// One BM-token x 256-weight-row tile. Each of the 8 waves streams its own 32 weight rows from HBM
// straight into MFMA A-operand registers (a weight row is used by one wave only, so it never touches
// LDS); the BM token rows, shared by all waves, are staged through double-buffered LDS. Per 64-wide K
// step a lane loads 32 contiguous bytes of each of its 2 weight rows (k-group g = lane / 16 covers
// k 16 g .. 16 g + 15); MFMA h in {0, 1} takes the h-th 8 of them and token chunk 2 g + h from LDS.
// With 8 waves the register budget allows two waves per SIMD, so one wave's memory waits are covered by
// the other's MFMAs.
// Pipeline: step s computes on weights W(s) (register set s % 3) and tokens X(s) (LDS buffer s % 2). It
// first issues the token loads of X(s + XS) and the weight loads of W(s + 2) (into registers whose last
// use is over); at its end it stores X(s + 1) into LDS buffer (s + 1) % 2, whose last reader was step
// s - 1, and a barrier publishes it. Loads past the end re-read the last chunk (in bounds, unused); the
// scheduling barrier keeps each step's loads ahead of its MFMAs.
// Only NB of the token blocks (the ones holding valid rows, rounded up to a compiled count: any count at
// BM 128, an even one at BM 256, a power of two for dense tiles) are computed.
template <GemmKind KIND, bool DENSE, int BM, int NB>
__device__ __forceinline__ void wide_tile(const GemmArgs& a, const TileInfo& ti, int split, int col0,
                                          const uint16_t* const (&wsrc)[2],
                                          const uint16_t* const (&xsrc)[WideShape<BM>::XQ], int kbeg, int kend,
                                          uint16_t* xs0, uint16_t* xs1) {
    constexpr int XQ = WideShape<BM>::XQ, XS = WideShape<BM>::XS, G = WideShape<BM>::G;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int rl = lane & 15, kg = lane >> 4;
    const int lc = tid & 7;
    const int N = a.N;

    f32x4 acc[2][NB];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    typedef Pack16 WSet[2][2];
    typedef Pack16 XSet[XQ];
    WSet w0, w1, w2;
    XSet xa, xb;
    XSet& xA = xa;
    XSet& xB = XS == 2 ? xb : xa; // with one stage the load and store sets are the same registers
    auto wload = [&](WSet& w, int kk) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            w[i][0] = load16(wsrc[i] + kk);
            w[i][1] = load16(wsrc[i] + kk + 8);
        }
    };
    auto xload = [&](XSet& x, int kk) {
#pragma unroll
        for (int q = 0; q < XQ; ++q) x[q] = load16(xsrc[q] + kk);
    };
    auto xstore = [&](const XSet& x, uint16_t* buf) {
#pragma unroll
        for (int q = 0; q < XQ; ++q) store16(&buf[lds_off((tid >> 3) + 64 * q, lc)], x[q]);
    };
    // Token fragments, G blocks at a time: the group's first-half fragments are read up front; each
    // second-half fragment is read into the register its first-half twin frees, right after that twin's
    // MFMAs issue.
    auto compute = [&](const WSet& w, const uint16_t* xb_lds) {
#pragma unroll
        for (int c0 = 0; c0 < NB; c0 += G) {
            Pack16 bfr[G];
#pragma unroll
            for (int jj = 0; jj < G; ++jj)
                if (c0 + jj < NB) bfr[jj] = load16(&xb_lds[lds_off((c0 + jj) * 16 + rl, 2 * kg)]);
#pragma unroll
            for (int jj = 0; jj < G; ++jj)
                if (c0 + jj < NB) {
#pragma unroll
                    for (int i = 0; i < 2; ++i)
                        acc[i][c0 + jj] = mfma16x16x32(w[i][0], bfr[jj], acc[i][c0 + jj]);
                    bfr[jj] = load16(&xb_lds[lds_off((c0 + jj) * 16 + rl, 2 * kg + 1)]);
                }
#pragma unroll
            for (int jj = 0; jj < G; ++jj)
                if (c0 + jj < NB) {
#pragma unroll
                    for (int i = 0; i < 2; ++i)
                        acc[i][c0 + jj] = mfma16x16x32(w[i][1], bfr[jj], acc[i][c0 + jj]);
                }
        }
    };

    const int nk = (kend - kbeg) / kBK;
    const int klast = kend - kBK;
    auto kat = [&](int st) { const int k = kbeg + st * kBK; return k < klast ? k : klast; };
    auto step = [&](const WSet& wcur, WSet& wfut, XSet& xfut, const XSet& xnext, const uint16_t* bcur,
                    uint16_t* bnext, int st) {
        xload(xfut, kat(st + XS));
        wload(wfut, kat(st + 2));
        __builtin_amdgcn_sched_barrier(0);
        compute(wcur, bcur);
        xstore(xnext, bnext);
        __syncthreads();
    };
    xload(xA, kat(0));
    wload(w0, kat(0));
    if (XS == 2) xload(xB, kat(1));
    wload(w1, kat(1));
    xstore(xA, xs0);
    __syncthreads();
    // six steps per iteration: the weight registers cycle with period 3, the token sets and LDS buffers
    // with period 2
    int s = 0;
    for (; s + 6 <= nk; s += 6) {
        step(w0, w2, xA, xB, xs0, xs1, s);
        step(w1, w0, xB, xA, xs1, xs0, s + 1);
        step(w2, w1, xA, xB, xs0, xs1, s + 2);
        step(w0, w2, xB, xA, xs1, xs0, s + 3);
        step(w1, w0, xA, xB, xs0, xs1, s + 4);
        step(w2, w1, xB, xA, xs1, xs0, s + 5);
    }
    if (s < nk) step(w0, w2, xA, xB, xs0, xs1, s);
    if (s + 1 < nk) step(w1, w0, xB, xA, xs1, xs0, s + 1);
    if (s + 2 < nk) step(w2, w1, xA, xB, xs0, xs1, s + 2);
    if (s + 3 < nk) step(w0, w2, xB, xA, xs1, xs0, s + 3);
    if (s + 4 < nk) step(w1, w0, xA, xB, xs0, xs1, s + 4);
    if (col0 >= N) return; // a wave past the last output column computed on clamped rows: nothing to store

    // epilogue: lane holds features 4 kg + r of weight block i and token rl of token block j
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const int m = j * 16 + rl;
        if (m >= ti.rows) continue;
        const size_t row = (size_t)ti.off + ti.m0 + m;
        if (KIND == GemmKind::GateUp) {
            const int col = col0 + 4 * kg;
            const f32x4 g = acc[0][j], u = acc[1][j];
            uint2 v;
            v.x = pack_bf16x2(swiglu(g[0], u[0]), swiglu(g[1], u[1]));
            v.y = pack_bf16x2(swiglu(g[2], u[2]), swiglu(g[3], u[3]));
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + row * N + col) = v;
        } else {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int col = col0 + i * 16 + 4 * kg;
                if (col >= N) continue;
                const f32x4 y = acc[i][j];
                if (KIND == GemmKind::DownF32 && !DENSE && a.out_bf16) { // per-slot rows as bf16 (N % 64 == 0)
                    uint2 v;
                    v.x = pack_bf16x2(y[0], y[1]);
                    v.y = pack_bf16x2(y[2], y[3]);
                    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + row * N + col) = v;
                    continue;
                }
                float* o = static_cast<float*>(a.out) + (size_t)split * a.dense_rows * N + row * N + col;
                if (col + 3 < N) {
                    *reinterpret_cast<float4*>(o) = make_float4(y[0], y[1], y[2], y[3]);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (col + r < N) o[r] = y[r];
                }
            }
        }
    }
}

template <GemmKind KIND, bool DENSE, int BM>
__global__ __launch_bounds__(kWThreads) void gemm_wide_kernel(GemmArgs a, int ntn, int64_t tiles_per_split) {
    constexpr int XQ = WideShape<BM>::XQ;
    int64_t bid = blockIdx.x;
    int split = 0;
    if (KIND == GemmKind::Logits) {
        split = (int)(bid / (tiles_per_split * ntn));
        bid -= (int64_t)split * tiles_per_split * ntn;
    }
    int ntile;
    TileInfo ti;
    if (DENSE) {
        ntile = (int)(bid % ntn);
        if (!tile_info<true, BM>(a, bid / ntn, ti)) return;
    } else if (!grouped_block<BM>(a, ntn, bid, ti, ntile)) {
        return;
    }

    __shared__ __attribute__((aligned(16))) uint16_t xs0[BM * kBK];
    __shared__ __attribute__((aligned(16))) uint16_t xs1[BM * kBK];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int rl = lane & 15, kg = lane >> 4;
    const int K = a.K, N = a.N;

    int kbeg = 0, kend = K;
    if (KIND == GemmKind::Logits) {
        const int C = K / kBK;
        kbeg = (int)((int64_t)split * C / a.ksplit) * kBK;
        kend = (int)((int64_t)(split + 1) * C / a.ksplit) * kBK;
    }

    // this wave's two weight row blocks, clamped to the last row (a wave past N computes on them and
    // stores nothing). Gate/up: W1 and W3 rows of the same 16 output columns.
    int col0;
    const uint16_t* wsrc[2];
    if (KIND == GemmKind::GateUp) {
        col0 = ntile * (kWBN / 2) + wave * 16;
        int n = col0 + rl;
        n = n < N ? n : N - 1;
        wsrc[0] = weight_row(a.w_a, a.ws_a, ti, N, n, K) + kg * 16;
        wsrc[1] = weight_row(a.w_b, a.ws_b, ti, N, n, K) + kg * 16;
    } else {
        col0 = ntile * kWBN + wave * kWaveRows;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            int n = col0 + i * 16 + rl;
            n = n < N ? n : N - 1;
            wsrc[i] = weight_row(a.w_a, a.ws_a, ti, N, n, K) + kg * 16;
        }
    }
    const int lc = tid & 7;
    const uint16_t* xsrc[XQ];
#pragma unroll
    for (int q = 0; q < XQ; ++q) xsrc[q] = act_row<KIND, DENSE>(a, ti, (tid >> 3) + 64 * q) + lc * 8;

    const int nbj = (ti.rows + 15) >> 4;
#define MOE_WIDE_TILE(NBV) wide_tile<KIND, DENSE, BM, NBV>(a, ti, split, col0, wsrc, xsrc, kbeg, kend, xs0, xs1)
    if constexpr (DENSE) {
        // dense tiles are full but for the last: power-of-two block counts
        if (nbj > BM / 32) MOE_WIDE_TILE(BM / 16);
        else if (nbj > 4) MOE_WIDE_TILE(8);
        else if (nbj > 2) MOE_WIDE_TILE(4);
        else if (nbj > 1) MOE_WIDE_TILE(2);
        else MOE_WIDE_TILE(1);
    } else if constexpr (BM == kTallBM) {
        // tile heights are multiples of 32 rows: even block counts (a shorter last tile rounds up)
        if (nbj > 14) MOE_WIDE_TILE(16);
        else if (nbj > 12) MOE_WIDE_TILE(14);
        else if (nbj > 10) MOE_WIDE_TILE(12);
        else if (nbj > 8) MOE_WIDE_TILE(10);
        else if (nbj > 6) MOE_WIDE_TILE(8);
        else if (nbj > 4) MOE_WIDE_TILE(6);
        else if (nbj > 2) MOE_WIDE_TILE(4);
        else if (nbj > 1) MOE_WIDE_TILE(2);
        else MOE_WIDE_TILE(1);
    } else {
        switch (nbj) {
        case 1: MOE_WIDE_TILE(1); break;
        case 2: MOE_WIDE_TILE(2); break;
        case 3: MOE_WIDE_TILE(3); break;
        case 4: MOE_WIDE_TILE(4); break;
        case 5: MOE_WIDE_TILE(5); break;
        case 6: MOE_WIDE_TILE(6); break;
        case 7: MOE_WIDE_TILE(7); break;
        default: MOE_WIDE_TILE(8); break;
        }
    }
#undef MOE_WIDE_TILE
}

// ------------------------------------------------------------------------------------------------
// dma kernel

// Loads into VGPRs reach about 16 B/clk per CU from L2; copies straight into LDS (buffer loads to LDS, 16
// bytes per lane) about 50. So both operands of a 256 x 256 tile go through LDS this way. Wave
// (wm = wave % 4, wn = wave / 4) computes 64 weight rows (gate/up: 32 features of W1 and the same 32 of
// W3) x the token blocks 2 jj + wn, from 16-byte LDS fragments; each accumulator sums its products in
// the same order as the wide kernel's, so both give the same bits.
constexpr int kDThreads = 512;
constexpr int kDRows = 256; // weight rows and token rows per tile

typedef __attribute__((address_space(3))) void* lptr_t;

// Raw buffer resource over 4 GiB from `base` (stride 0, 32-bit offsets; word 3 as gfx9-family raw buffers
// take it).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dma_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)0xFFFFFFFF, 0x00020000);
}

// LDS layout of both operands: [256 rows][64 k] bf16, 16-byte chunk c of row r at slot c ^ dswz(r) (the
// wide kernel's swizzle: conflict-free fragment reads).
__device__ __forceinline__ int dswz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// Blocks [lo, hi) of the expert-major order that XCD x takes: the work-balanced split when the permutation
// wrote one, else contiguous equal counts (the order grouped_block gives).
__device__ __forceinline__ void xcd_range(const GemmArgs& a, int ntn, int x, int& lo, int& hi) {
    if (a.xcd_bounds != nullptr) {
        lo = a.xcd_bounds[x];
        hi = a.xcd_bounds[x + 1];
        return;
    }
    const int live = a.ntiles[0] * ntn, chunk = (live + kXcds - 1) / kXcds;
    lo = min(x * chunk, live);
    hi = min(lo + chunk, live);
}

// The block a persistent workgroup of XCD x takes next (thread 0), or -1 when none is left: the front of its
// own XCD's range, then the back of the other XCDs' ranges (the blocks their own workgroups would reach
// last), through the counters of claim_block.
// With `home_old` (>= 0: what an earlier front claim on the own XCD's counter returned) the own range is
// decided from it and only the other XCDs' counters are tried.
__device__ __forceinline__ int grab_block(const GemmArgs& a, int ntn, int x, long long home_old = -1) {
    for (int d = 0; d < kXcds; ++d) {
        const int y = (x + d) % kXcds;
        int lo, hi;
        xcd_range(a, ntn, y, lo, hi);
        if (lo >= hi) continue;
        const unsigned long long old = d == 0 && home_old >= 0
                                           ? (unsigned long long)home_old
                                           : atomicAdd(a.work_ctr + y, d == 0 ? kClaimFront : kClaimBack);
        const int64_t c = claim_block(lo, hi, old, d == 0);
        if (c >= 0) return (int)c;
    }
    return -1;
}

// One tile of the DMA GEMM. Persistent kernel (PERSIST): `wave0` is the wave index (a scalar); after the
// tile's stores thread 0 claims the workgroup's next block, which wave 0 holds in `got` (-1: none left). With a K
// split S of 2 (decode-sized gate/up launches) the tile computes K range `ks` and writes fp32 partials of g
// and u instead of h.
// DEEP (tiles of at most 32 rows, decode): rings of four weight buffers and four token buffers of 64 rows
// (ws3, xs3 and the small xs0..xs3), so both operands are copied three K steps ahead: half again as many
// bytes in flight per CU as the two-ahead ring, which is what bounds a CU's weight stream at decode.
template <GemmKind KIND, bool DENSE, int NBW, bool PERSIST, bool DEEP = false>
__device__ __forceinline__ void dma_tile(const GemmArgs& a, const TileInfo& ti, int ntile, uint16_t* ws0,
                                         uint16_t* ws1, uint16_t* ws2, uint16_t* xs0, uint16_t* xs1, int wave0,
                                         int ntn, int& got, int ks = 0, int S = 1, uint16_t* ws3 = nullptr,
                                         uint16_t* xs2 = nullptr, uint16_t* xs3 = nullptr) {
    static_assert(!DEEP || (NBW == 1 && !PERSIST), "the deep ring holds 64 token rows, one-shot tiles only");
    constexpr int XI = (NBW + 1) / 2; // token load instructions per wave and K step
    // persistent: the lane index comes from mbcnt, so nothing derived from the thread index has to stay in
    // registers from one tile to the next
    const int lane =
        PERSIST ? (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) : (int)(threadIdx.x & 63);
    const int wave = PERSIST ? wave0 : __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tid = wave * 64 + lane;
    const int rl = lane & 15, kg = lane >> 4;
    const int wm = wave & 3, wn = wave >> 2;
    const int K = a.K, N = a.N;
    // K steps [sb, sb + nk) of the nk_all: all of them, or half with a K split of 2
    const int nk_all = K / kBK;
    const int sb = ks * nk_all / S;
    const int nk = (ks + 1) * nk_all / S - sb;

    // Load instruction t (8 rows = 1 KB of LDS) of an operand is issued by wave t % 8: 4 weight loads and
    // XI token loads per wave and step (token rows past the computed blocks are not loaded, but for an odd
    // instruction's, which clamp to the tile's rows). Lane l fills slot l % 8 of row 8 t + l / 8 with
    // global chunk (l % 8) ^ dswz(row). Addresses: a wave-uniform base plus a 32-bit per-lane byte offset.
    const int lr = lane >> 3, ls = lane & 7;
    const char* wbase0 = reinterpret_cast<const char*>(weight_row(a.w_a, a.ws_a, ti, N, 0, K));
    const char* wbase1 =
        KIND == GemmKind::GateUp ? reinterpret_cast<const char*>(weight_row(a.w_b, a.ws_b, ti, N, 0, K)) : wbase0;
    const char* xbase = reinterpret_cast<const char*>(a.act);
    uint32_t woff[4], xoff[XI];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int r = 8 * (wave + 8 * q) + lr;
        // gate/up: LDS weight rows 0..127 are W1 rows (instructions 0..15), 128..255 the same W3 rows
        int n = KIND == GemmKind::GateUp ? ntile * 128 + (r & 127) : ntile * 256 + r;
        n = n < N ? n : N - 1;
        woff[q] = (uint32_t)n * (uint32_t)K * 2u + (uint32_t)(ls ^ dswz(r)) * 16u;
    }
#pragma unroll
    for (int q = 0; q < XI; ++q) {
        const int r = 8 * (wave + 8 * q) + lr;
        xoff[q] = (uint32_t)(reinterpret_cast<const char*>(act_row<KIND, DENSE>(a, ti, r)) - xbase) +
                  (uint32_t)(ls ^ dswz(r)) * 16u;
    }
    // The copies are raw buffer loads: the per-lane offsets stay fixed 32-bit registers and the K step goes
    // into the scalar offset (no per-lane 64-bit addresses to advance).
    const __amdgpu_buffer_rsrc_t rx = dma_rsrc(xbase), rw0 = dma_rsrc(wbase0),
                                 rw1 = KIND == GemmKind::GateUp ? dma_rsrc(wbase1) : rw0;
    auto load_x = [&](uint16_t* xl, int st) {
#pragma unroll
        for (int q = 0; q < XI; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lptr_t)(xl + 8 * (wave + 8 * q) * kBK), 16, xoff[q],
                                                     2 * (sb + st) * kBK, 0, 0);
    };
    auto load_w = [&](uint16_t* wl, int st) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(KIND == GemmKind::GateUp && q >= 2 ? rw1 : rw0,
                                                     (lptr_t)(wl + 8 * (wave + 8 * q) * kBK), 16, woff[q],
                                                     2 * (sb + st) * kBK, 0, 0);
    };

    // fragments: block bases are multiples of 16 rows, so the swizzle depends on the lane only
    auto arow = [&](int i) {
        if (KIND == GemmKind::GateUp) return (i < 2 ? 0 : 128) + 32 * wm + 16 * (i & 1);
        return 64 * wm + 16 * i;
    };
    auto brow = [&](int jj) { return 16 * (2 * jj + wn); };
    const int lo0 = rl * kBK + (((2 * kg) ^ dswz(rl)) << 3), lo1 = rl * kBK + (((2 * kg + 1) ^ dswz(rl)) << 3);
    auto frag = [&](const uint16_t* l, int row0, int h) { return load16(&l[row0 * kBK + (h ? lo1 : lo0)]); };

    f32x4 acc[4][NBW];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NBW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    Pack16 f0a[4], f0b[NBW], f1a[4], f1b[NBW]; // fragments of the two K halves of a step
    auto read = [&](Pack16 (&fa)[4], Pack16 (&fb)[NBW], const uint16_t* wl, const uint16_t* xl, int h) {
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[i] = frag(wl, arow(i), h);
#pragma unroll
        for (int j = 0; j < NBW; ++j) fb[j] = frag(xl, brow(j), h);
    };
    auto mma = [&](const Pack16 (&fa)[4], const Pack16 (&fb)[NBW]) {
#pragma unroll
        for (int j = 0; j < NBW; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i][j] = mfma16x16x32(fa[i], fb[j], acc[i][j]);
    };
    // the fragment reads of one half spread evenly among the other half's MFMAs
    auto interleave = [&]() {
        constexpr int R = 4 + NBW, M = 4 * NBW, Q = M / R;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            __builtin_amdgcn_sched_group_barrier(0x008, Q, 0); // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); // LDS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, M - Q * R, 0);
        __builtin_amdgcn_sched_barrier(0);
    };

    // Pipeline. Weights go into a ring of three LDS buffers (step s in ws[s % 3]), tokens into two
    // (xs[s % 2]). Step s: read the second-half fragments of step s, MFMAs of its first half; then the
    // barrier that opens step s + 1: each wave first waits until at most its 4 youngest loads (the
    // weights of step s + 2) are in flight, so after the barrier step s + 1 is in LDS for everyone and
    // nobody reads step s's buffers any more; the tokens of step s + 2 and the weights of step s + 3 go
    // into those buffers; then the MFMAs of step s's second half, with the first-half fragments of step
    // s + 1 read among them. Weights are thus loaded two steps ahead, tokens one. Copies of steps past the
    // last one repeat the last step (data the workgroup has just read, so they come from L2, and nobody
    // reads them): every step runs the same branch-free code, which keeps the compiler from adding waits or
    // spills of its own around conditional copies.
    // Persistent form: thread 0 sends the front claim on its own XCD's counter before the tile's last K
    // steps (an unconditional add: a claim on an empty or used-up range just gets no block), so its round
    // trip overlaps them; the tile's end decides from the value it returned. Gate/up sends it at the start
    // of the last full six-step iteration, down (whose loop has no register to spare) after that loop.
    long long home_old = -1;
    auto early_claim = [&]() {
        if constexpr (PERSIST)
            if (tid == 0) home_old = (long long)atomicAdd(a.work_ctr + (int)(blockIdx.x % kXcds), kClaimFront);
    };
    auto step = [&](uint16_t* wc, uint16_t* xc, const uint16_t* wn1, const uint16_t* xn1, int s) {
        read(f1a, f1b, wc, xc, 1);
        mma(f0a, f0b);
        interleave();
        __builtin_amdgcn_s_waitcnt(0x0074); // vmcnt(4) lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        load_x(xc, min(s + 2, nk - 1));
        __builtin_amdgcn_sched_barrier(0); // the weights must be the youngest copies (the vmcnt(4) above)
        load_w(wc, min(s + 3, nk - 1));
        __builtin_amdgcn_sched_barrier(0);
        read(f0a, f0b, wn1, xn1, 0);
        mma(f1a, f1b);
        interleave();
    };
    // Prologue: every buffer is free at the start of a tile, so steps 0 and 1 (and the weights of step 2)
    // are requested at once, in the order X0 W0 X1 W1 W2; the barrier that opens step 0 waits for X0 and W0
    // only (the 4 XI + 8 younger copies may stay in flight), the one that opens step 1 (inside step 0)
    // for X1 and W1 (W2 may stay in flight), as in every later step. With fewer than three K steps the
    // copies of steps past the last one repeat the last step (unread; the end of the tile waits for them):
    // one branch-free sequence lets the compiler see that the first reads need X0 and W0 only.
    if constexpr (!DEEP) {
        constexpr int V2 = XI + 8;
        static_assert(V2 <= 15, "vmcnt immediates below hold 4 bits");
        load_x(xs0, 0);
        __builtin_amdgcn_sched_barrier(0);
        load_w(ws0, 0);
        __builtin_amdgcn_sched_barrier(0);
        load_x(xs1, min(1, nk - 1));
        __builtin_amdgcn_sched_barrier(0);
        load_w(ws1, min(1, nk - 1));
        __builtin_amdgcn_sched_barrier(0);
        load_w(ws2, min(2, nk - 1));
        __builtin_amdgcn_s_waitcnt(0x0070 | V2); // vmcnt(XI + 8) lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        read(f0a, f0b, ws0, xs0, 0);
        // six steps per iteration (weight buffers cycle with period 3, token buffers with 2), then up to five
        int s = 0;
        for (; s + 6 <= nk; s += 6) {
            if (KIND == GemmKind::GateUp && s + 12 > nk) early_claim();
            step(ws0, xs0, ws1, xs1, s);
            step(ws1, xs1, ws2, xs0, s + 1);
            step(ws2, xs0, ws0, xs1, s + 2);
            step(ws0, xs1, ws1, xs0, s + 3);
            step(ws1, xs0, ws2, xs1, s + 4);
            step(ws2, xs1, ws0, xs0, s + 5);
        }
        if (KIND != GemmKind::GateUp || nk < 6) early_claim();
        if (s < nk) step(ws0, xs0, ws1, xs1, s);
        if (s + 1 < nk) step(ws1, xs1, ws2, xs0, s + 1);
        if (s + 2 < nk) step(ws2, xs0, ws0, xs1, s + 2);
        if (s + 3 < nk) step(ws0, xs1, ws1, xs0, s + 3);
        if (s + 4 < nk) step(ws1, xs0, ws2, xs1, s + 4);
    } else {
        // Deep ring: W(s) in ws[s % 4], X(s) in xs[s % 4]. Step s, after its barrier, copies X(s + 4) and
        // W(s + 4) into the buffers of X(s) and W(s); the barrier that opens step s + 1 waits for X(s + 1) and
        // W(s + 1), while the copies of steps s + 2 and s + 3 may stay in flight.
        constexpr int VD = 2 * (XI + 4), VP = 3 * (XI + 4);
        static_assert(VP <= 15, "vmcnt immediates below hold 4 bits");
        auto dstep = [&](uint16_t* wc, uint16_t* xc, const uint16_t* wn1, const uint16_t* xn1, int s) {
            read(f1a, f1b, wc, xc, 1);
            mma(f0a, f0b);
            interleave();
            __builtin_amdgcn_s_waitcnt(0x0070 | VD); // vmcnt(2 (XI + 4)) lgkmcnt(0)
            __builtin_amdgcn_s_barrier();
            load_x(xc, min(s + 4, nk - 1));
            __builtin_amdgcn_sched_barrier(0);
            load_w(wc, min(s + 4, nk - 1));
            __builtin_amdgcn_sched_barrier(0);
            read(f0a, f0b, wn1, xn1, 0);
            mma(f1a, f1b);
            interleave();
        };
        // prologue: steps 0 to 3; the first barrier waits for X0 and W0
        load_x(xs0, 0);
        __builtin_amdgcn_sched_barrier(0);
        load_w(ws0, 0);
        __builtin_amdgcn_sched_barrier(0);
        load_x(xs1, min(1, nk - 1));
        __builtin_amdgcn_sched_barrier(0);
        load_w(ws1, min(1, nk - 1));
        __builtin_amdgcn_sched_barrier(0);
        load_x(xs2, min(2, nk - 1));
        __builtin_amdgcn_sched_barrier(0);
        load_w(ws2, min(2, nk - 1));
        __builtin_amdgcn_sched_barrier(0);
        load_x(xs3, min(3, nk - 1));
        __builtin_amdgcn_sched_barrier(0);
        load_w(ws3, min(3, nk - 1));
        __builtin_amdgcn_s_waitcnt(0x0070 | VP); // vmcnt(3 (XI + 4)) lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        read(f0a, f0b, ws0, xs0, 0);
        // four steps per iteration, then up to three (none when the K steps are a multiple of four)
        int s = 0;
        for (; s + 4 <= nk; s += 4) {
            dstep(ws0, xs0, ws1, xs1, s);
            dstep(ws1, xs1, ws2, xs2, s + 1);
            dstep(ws2, xs2, ws3, xs3, s + 2);
            dstep(ws3, xs3, ws0, xs0, s + 3);
        }
        if (s < nk) dstep(ws0, xs0, ws1, xs1, s);
        if (s + 1 < nk) dstep(ws1, xs1, ws2, xs2, s + 1);
        if (s + 2 < nk) dstep(ws2, xs2, ws3, xs3, s + 2);
    }
    __builtin_amdgcn_s_waitcnt(0x0070); // no copy into LDS may outlive the workgroup
    // persistent form: thread 0 claims the next block once the tile's stores are issued, so the claim's round
    // trip overlaps their drain
    auto claim_next = [&]() {
        if constexpr (PERSIST) {
            int claim = -1;
            if (tid == 0) claim = grab_block(a, ntn, (int)(blockIdx.x % kXcds), home_old);
            if (wave == 0) got = __builtin_amdgcn_readfirstlane(claim);
        }
    };

    if constexpr (KIND == GemmKind::DownF32) {
        // rows leave through LDS: each wave turns one 16-token block at a time into 16 rows of its 64
        // features in a private 4.25 KB area of ws0 / ws1 (fp32, row stride 68 floats), then stores whole
        // row segments (256 contiguous bytes per fp32 row, 128 per bf16 row)
        __syncthreads(); // every wave is done reading the operand buffers
        float* stg = reinterpret_cast<float*>(wave < 4 ? ws0 : ws1) + (wave & 3) * (16 * 68);
        const int c4 = lane & 15, r4 = lane >> 4;
        const int colw = ntile * 256 + 64 * wm;
        // K split: the rows of ranges 2 .. S go to the partial buffers, the combine adds them. A folded
        // shared expert with rows of its own writes fp32 rows there, indexed by token.
        const bool own = !DENSE && ti.shared && a.out_shared != nullptr;
        float* yout = own ? a.out_shared
                          : DENSE && S > 1 ? a.part + (size_t)ks * a.part_rows * N // every range writes a partial
                                           : (ks == 0 ? static_cast<float*>(a.out)
                                                      : a.part + (size_t)(ks - 1) * a.part_rows * N);
        const size_t row0 = own ? (size_t)ti.m0 : (size_t)ti.off + ti.m0;
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<f32x4*>(stg + rl * 68 + 16 * i + 4 * kg) = acc[i][j];
            __builtin_amdgcn_s_waitcnt(0xC07F); // lgkmcnt(0): the block is in LDS
            if (!DENSE && a.out_bf16 && !own) {
                // bf16 rows (N % 64 == 0, no K split): 8 lanes of 16 bytes per row segment, 8 rows per store
                const int c8 = lane & 7, r8 = lane >> 3;
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    const int t = 8 * p + r8;
                    const f32x4 v0 = *reinterpret_cast<const f32x4*>(stg + t * 68 + 8 * c8);
                    const f32x4 v1 = *reinterpret_cast<const f32x4*>(stg + t * 68 + 8 * c8 + 4);
                    const int m = 16 * (2 * j + wn) + t;
                    const int col = colw + 8 * c8;
                    if (m < ti.rows && col < N) {
                        Pack16 q;
                        q.w[0] = pack_bf16x2(v0[0], v0[1]);
                        q.w[1] = pack_bf16x2(v0[2], v0[3]);
                        q.w[2] = pack_bf16x2(v1[0], v1[1]);
                        q.w[3] = pack_bf16x2(v1[2], v1[3]);
                        store16(static_cast<uint16_t*>(a.out) + ((size_t)ti.off + ti.m0 + m) * N + col, q);
                    }
                }
            } else {
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const int t = 4 * p + r4;
                    const f32x4 v = *reinterpret_cast<const f32x4*>(stg + t * 68 + 4 * c4);
                    const int m = 16 * (2 * j + wn) + t;
                    const int col = colw + 4 * c4;
                    if (m < ti.rows && col < N) *reinterpret_cast<f32x4*>(yout + (row0 + m) * N + col) = v;
                }
            }
            __builtin_amdgcn_s_waitcnt(0xC07F); // reads done before the next block overwrites the area
        }
    } else {
        // gate/up: lane holds features 4 kg + r of weight blocks i (g) and i + 2 (u), token rl of token
        // block 2 jj + wn
        static_assert(KIND == GemmKind::GateUp, "the dma kernel computes gate/up and fp32 down GEMMs");
        if (S > 1) {
            // K split: fp32 partials of g (columns [0, N)) and u ([N, 2N)) of this K range
            float* part = a.part + (size_t)ks * a.part_rows * 2 * N;
#pragma unroll
            for (int j = 0; j < NBW; ++j) {
                const int m = 16 * (2 * j + wn) + rl;
                if (m >= ti.rows) continue;
                float* prow = part + ((size_t)ti.off + ti.m0 + m) * 2 * N;
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int col = ntile * 128 + 32 * wm + 16 * i + 4 * kg;
                    if (col >= N) continue;
                    *reinterpret_cast<f32x4*>(prow + col) = acc[i][j];
                    *reinterpret_cast<f32x4*>(prow + N + col) = acc[i + 2][j];
                }
            }
            claim_next();
            return;
        }
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
            const int m = 16 * (2 * j + wn) + rl;
            if (m >= ti.rows) continue;
            const size_t row = (size_t)ti.off + ti.m0 + m;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int col = ntile * 128 + 32 * wm + 16 * i + 4 * kg;
                if (col >= N) continue;
                const f32x4 g = acc[i][j], u = acc[i + 2][j];
                uint2 v;
                v.x = pack_bf16x2(swiglu(g[0], u[0]), swiglu(g[1], u[1]));
                v.y = pack_bf16x2(swiglu(g[2], u[2]), swiglu(g[3], u[3]));
                *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + row * N + col) = v;
            }
        }
    }
    claim_next();
}

template <GemmKind KIND, bool DENSE>
__global__ __launch_bounds__(kDThreads) void gemm_dma_kernel(GemmArgs a, int ntn) {
    int64_t bid = blockIdx.x;
    int ntile, S = 1, ks = 0;
    if (!DENSE && KIND != GemmKind::Logits && a.ksplit_dev != nullptr) S = device_split(a.ksplit_dev);
    if (DENSE && a.ksplit > 1) { // dense, few rows: the grid is the K ranges times the blocks of one range
        S = a.ksplit;
        const int64_t per = (int64_t)((a.dense_rows + kDRows - 1) / kDRows) * ntn;
        ks = (int)(bid / per);
        if (ks >= S) return;
        bid -= (int64_t)ks * per;
    }
    TileInfo ti;
    if (DENSE) {
        ntile = (int)(bid % ntn);
        if (!tile_info<true, kDRows>(a, bid / ntn, ti)) return;
    } else if (a.xcd_bounds != nullptr ? !balanced_block<kDRows>(a, ntn, bid, ti, ntile)
                                       : !grouped_block<kDRows>(a, ntn, bid, ti, ntile, S, &ks)) {
        return;
    }

    // 160 KB: three weight buffers and two token buffers of [256][64] bf16
    __shared__ __attribute__((aligned(16))) uint16_t ws0[kDRows * kBK];
    __shared__ __attribute__((aligned(16))) uint16_t ws1[kDRows * kBK];
    __shared__ __attribute__((aligned(16))) uint16_t ws2[kDRows * kBK];
    __shared__ __attribute__((aligned(16))) uint16_t xs0[kDRows * kBK];
    __shared__ __attribute__((aligned(16))) uint16_t xs1[kDRows * kBK];

    // 16-row token blocks per wave: tiles up to 256 rows, 32 per pair of token waves
    const int nb = (ti.rows + 31) >> 5;
    int got = 0;
#define MOE_DMA_TILE(NBV) dma_tile<KIND, DENSE, NBV, false>(a, ti, ntile, ws0, ws1, ws2, xs0, xs1, 0, ntn, got, ks, S)
    switch (nb) {
    case 1: MOE_DMA_TILE(1); break;
    case 2: MOE_DMA_TILE(2); break;
    case 3: MOE_DMA_TILE(3); break;
    case 4: MOE_DMA_TILE(4); break;
    case 5: MOE_DMA_TILE(5); break;
    case 6: MOE_DMA_TILE(6); break;
    case 7: MOE_DMA_TILE(7); break;
    default: MOE_DMA_TILE(8); break;
    }
#undef MOE_DMA_TILE
}


// The same one-shot GEMM for launches whose tiles all hold at most 32 rows (decode sizes): the deep ring of
// dma_tile (four 32 KB weight buffers, four 8 KB token buffers of 64 rows: 160 KB).
template <GemmKind KIND, bool DENSE>
__global__ __launch_bounds__(kDThreads) void gemm_dma_deep_kernel(GemmArgs a, int ntn) {
    int64_t bid = blockIdx.x;
    int ntile, S = 1, ks = 0;
    if (!DENSE && KIND != GemmKind::Logits && a.ksplit_dev != nullptr) S = device_split(a.ksplit_dev);
    if (DENSE && a.ksplit > 1) {
        S = a.ksplit;
        const int64_t per = (int64_t)((a.dense_rows + kDRows - 1) / kDRows) * ntn;
        ks = (int)(bid / per);
        if (ks >= S) return;
        bid -= (int64_t)ks * per;
    }
    TileInfo ti;
    if (DENSE) {
        ntile = (int)(bid % ntn);
        if (!tile_info<true, kDRows>(a, bid / ntn, ti)) return;
    } else if (a.xcd_bounds != nullptr ? !balanced_block<kDRows>(a, ntn, bid, ti, ntile)
                                       : !grouped_block<kDRows>(a, ntn, bid, ti, ntile, S, &ks)) {
        return;
    }
    if (ti.rows > 32) return; // the host launches this kernel only when no tile can exceed 32 rows
    __shared__ __attribute__((aligned(16))) uint16_t ws0[kDRows * kBK];
    __shared__ __attribute__((aligned(16))) uint16_t ws1[kDRows * kBK];
    __shared__ __attribute__((aligned(16))) uint16_t ws2[kDRows * kBK];
    __shared__ __attribute__((aligned(16))) uint16_t ws3[kDRows * kBK];
    __shared__ __attribute__((aligned(16))) uint16_t xs0[64 * kBK];
    __shared__ __attribute__((aligned(16))) uint16_t xs1[64 * kBK];
    __shared__ __attribute__((aligned(16))) uint16_t xs2[64 * kBK];
    __shared__ __attribute__((aligned(16))) uint16_t xs3[64 * kBK];
    int got = 0;
    dma_tile<KIND, DENSE, 1, false, true>(a, ti, ntile, ws0, ws1, ws2, xs0, xs1, 0, ntn, got, ks, S, ws3, xs2, xs3);
}

// Decode-sized launches streamed: one workgroup per CU runs the blocks blockIdx.x, blockIdx.x + gridDim.x, ...
// of the one-shot kernel's order back to back with the deep ring, and the copies its last four K steps issue
// are the next block's first four steps (the one-shot kernel repeats its last step there), so the copy stream
// of a CU never pauses between blocks: no block starts with an empty ring. Every block has the same number of
// K steps, a multiple of the ring's period 4 (the host checks), so each block's step s lands in ws[s % 4]
// as in the one-shot kernel, whose bits each block reproduces. The tile list and the gate/up gather map are
// staged in LDS first: the next block's tile and its token rows are then read from LDS, never with a vector
// load that would have to wait behind the copies in flight. Waves 4-7 copy the same 32 token rows as waves
// 0-3 (a tile has at most 32 rows), which halves the token buffers and makes room for that staging; each
// wave still issues five copies per step, so the wait counts of the deep ring hold. The epilogue stores
// straight from the accumulators (every LDS buffer holds copies in flight by then). The loads of a wave
// return in order, so the stores it issues among its copies only make each wait stricter.
constexpr int kStreamMaxTiles = 320;  // tile-list entries staged (decode: one tile per group)
constexpr int kStreamMaxRows = 1024;  // row_token entries staged (T * k at T <= 32, k <= 32)

template <GemmKind KIND, bool DENSE>
__device__ __forceinline__ void dma_stream(const GemmArgs& a, int ntn, uint16_t* ws0, uint16_t* ws1, uint16_t* ws2,
                                           uint16_t* ws3, uint16_t* xs0, uint16_t* xs1, uint16_t* xs2, uint16_t* xs3,
                                           int* tl, int* rt) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tid = threadIdx.x;
    const int rl = lane & 15, kg = lane >> 4;
    const int wm = wave & 3, wn = wave >> 2;
    const int lr = lane >> 3, ls = lane & 7;
    const int K = a.K, N = a.N;
    const int nk_all = K / kBK;

    int S = 1;
    int64_t live;
    bool sk = false; // stream-K: this workgroup takes one contiguous share of every block's K steps
    int64_t p_end = 0;
    if (DENSE) {
        S = a.ksplit > 1 ? a.ksplit : 1;
        live = (int64_t)ntn * S; // at most 32 rows: one token tile
    } else {
        if (a.ksplit_dev != nullptr) {
            S = device_split(a.ksplit_dev);
            sk = S == 2 && a.ksplit_dev[2] == 1;
        }
        const int nt = min(a.ntiles[0], kStreamMaxTiles);
        for (int i = tid; i < nt; i += kDThreads) {
            const int4 e = a.tiles[i];
            tl[4 * i] = e.x;
            tl[4 * i + 1] = e.y;
            tl[4 * i + 2] = e.z;
            tl[4 * i + 3] = e.w;
        }
        if (KIND == GemmKind::GateUp)
            for (int i = tid; i < min(a.rt_rows, kStreamMaxRows); i += kDThreads) rt[i] = a.row_token[i];
        live = (int64_t)nt * ntn * S;
        // stream-K needs every block cut at most once (each workgroup's share at least one block: as many
        // blocks as workgroups) and whole ring periods; else the even split in two, which writes the same
        // two planes
        sk = sk && nk_all % 4 == 0 && (int64_t)nt * ntn >= (int64_t)gridDim.x && gridDim.x % kXcds == 0;
        __syncthreads();
    }
    const int nk = nk_all / S;

    // block v of the one-shot order: its tile, output-column tile and K range
    auto block_of = [&](int64_t v, TileInfo& ti, int& ntile, int& ks) -> bool {
        if (DENSE) {
            if (v >= live) return false;
            ks = (int)(v / ntn);
            ntile = (int)(v % ntn);
            ti.g = 0;
            ti.m0 = 0;
            ti.off = 0;
            ti.rows = min(32, a.dense_rows);
            ti.shared = false;
            return ti.rows > 0;
        }
        const int64_t L = xcd_block_order(v, live);
        if (L < 0) return false;
        ks = (int)(L % S);
        const int64_t Lb = L / S;
        const int* e = tl + 4 * (Lb / ntn);
        return block_from<kDRows>(a, ntn, Lb, make_int4(e[0], e[1], e[2], e[3]), ti, ntile) && ti.rows <= 32;
    };

    // A piece of work: K steps [sb, sb + n) of one block, written to partial plane `plane` (the K split's
    // range index); `zero`: the piece is a whole block of a stream-K launch, which also writes zeros to the
    // other plane (the reduction adds both planes of every row). `next` is the cursor of the piece after it.
    // Even split: the cursor is the one-shot block index v (the workgroup's blocks are v, v + grid, ...).
    // Stream-K: the cursor is a ring period (4 K steps) of the live blocks' periods in the one-shot order
    // without the XCD interleave, P per block; the workgroup in place `pos` takes periods
    // [pos T / G, (pos + 1) T / G) of the T in all, the places of one XCD's workgroups consecutive, so an
    // XCD's blocks are one contiguous run of the order, as with the even split. A block cut between two
    // workgroups gives its first piece plane 0 and its second plane 1.
    const int P = nk_all / 4;
    int64_t cursor = blockIdx.x;
    if (sk) {
        const int64_t G = gridDim.x, T4 = (live / S) * P;
        const int64_t pos = (int64_t)(blockIdx.x % kXcds) * (G / kXcds) + blockIdx.x / kXcds;
        cursor = pos * T4 / G;
        p_end = (pos + 1) * T4 / G;
    }
    struct Piece {
        TileInfo ti;
        int ntile, plane, sb, n;
        bool zero;
        int64_t next;
    };
    auto piece_at = [&](int64_t c, Piece& pc) -> bool {
        if (!sk) {
            if (!block_of(c, pc.ti, pc.ntile, pc.plane)) return false;
            pc.sb = pc.plane * nk;
            pc.n = nk;
            pc.zero = false;
            pc.next = c + gridDim.x;
            return true;
        }
        if (c >= p_end) return false;
        const int64_t Lb = c / P;
        const int ps = (int)(c - Lb * P);
        const int pe = (int)min((int64_t)P, p_end - Lb * P);
        const int* e = tl + 4 * (Lb / ntn);
        if (!block_from<kDRows>(a, ntn, Lb, make_int4(e[0], e[1], e[2], e[3]), pc.ti, pc.ntile) || pc.ti.rows > 32)
            return false;
        pc.plane = ps == 0 ? 0 : 1;
        pc.sb = 4 * ps;
        pc.n = 4 * (pe - ps);
        pc.zero = ps == 0 && pe == P;
        pc.next = Lb * P + pe;
        return true;
    };

    // copy source of a block: weight resources and per-lane offsets as in dma_tile, the token rows of waves
    // 4-7 those of waves 0-3
    struct Src {
        const uint16_t* w0;
        const uint16_t* w1;
        uint32_t woff[4];
        uint32_t xoff;
        int sb; // first K step of the block's range
    };
    auto source = [&](const TileInfo& ti, int ntile, int sb) {
        Src c;
        c.w0 = weight_row(a.w_a, a.ws_a, ti, N, 0, K);
        c.w1 = KIND == GemmKind::GateUp ? weight_row(a.w_b, a.ws_b, ti, N, 0, K) : c.w0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = 8 * (wave + 8 * q) + lr;
            int n = KIND == GemmKind::GateUp ? ntile * 128 + (r & 127) : ntile * 256 + r;
            n = n < N ? n : N - 1;
            c.woff[q] = (uint32_t)n * (uint32_t)K * 2u + (uint32_t)(ls ^ dswz(r)) * 16u;
        }
        const int r = 8 * wm + lr;
        const int m = r < ti.rows ? r : ti.rows - 1;
        int row = ti.off + ti.m0 + m;
        if (KIND == GemmKind::GateUp && !DENSE) row = ti.shared ? ti.m0 + m : rt[row];
        c.xoff = (uint32_t)row * (uint32_t)K * 2u + (uint32_t)(ls ^ dswz(r)) * 16u;
        c.sb = sb;
        return c;
    };
    auto copy = [&](const Src& c, uint16_t* wl, uint16_t* xl, int st) {
        const int so = 2 * (c.sb + st) * kBK;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(dma_rsrc(a.act), (lptr_t)(xl + 8 * wm * kBK), 16, c.xoff, so, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        const __amdgpu_buffer_rsrc_t r0 = dma_rsrc(c.w0), r1 = dma_rsrc(c.w1);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(KIND == GemmKind::GateUp && q >= 2 ? r1 : r0,
                                                     (lptr_t)(wl + 8 * (wave + 8 * q) * kBK), 16, c.woff[q], so,
                                                     0, 0);
        __builtin_amdgcn_sched_barrier(0);
    };

    auto arow = [&](int i) {
        if (KIND == GemmKind::GateUp) return (i < 2 ? 0 : 128) + 32 * wm + 16 * (i & 1);
        return 64 * wm + 16 * i;
    };
    const int brow = 16 * wn;
    const int lo0 = rl * kBK + (((2 * kg) ^ dswz(rl)) << 3), lo1 = rl * kBK + (((2 * kg + 1) ^ dswz(rl)) << 3);
    auto frag = [&](const uint16_t* l, int row0, int h) { return load16(&l[row0 * kBK + (h ? lo1 : lo0)]); };
    f32x4 acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    Pack16 f0a[4], f0b, f1a[4], f1b;
    auto read = [&](Pack16 (&fa)[4], Pack16& fb, const uint16_t* wl, const uint16_t* xl, int h) {
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[i] = frag(wl, arow(i), h);
        fb = frag(xl, brow, h);
    };
    auto mma = [&](const Pack16 (&fa)[4], const Pack16& fb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = mfma16x16x32(fa[i], fb, acc[i]);
    };
    auto interleave = [&]() { // dma_tile's order at one token block: the five fragment reads, then the MFMAs
#pragma unroll
        for (int r = 0; r < 5; ++r) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); // LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);                               // MFMA
        __builtin_amdgcn_sched_barrier(0);
    };
    // step s of the ring (buffers wc, xc), as in dma_tile's deep ring; the copy after its barrier refills
    // them with step `st` of source c
    constexpr int VD = 2 * 5, VP = 3 * 5;
    auto dstep = [&](uint16_t* wc, uint16_t* xc, const uint16_t* wn1, const uint16_t* xn1, const Src& c, int st) {
        read(f1a, f1b, wc, xc, 1);
        mma(f0a, f0b);
        interleave();
        __builtin_amdgcn_s_waitcnt(0x0070 | VD); // vmcnt(10) lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        copy(c, wc, xc, st);
        read(f0a, f0b, wn1, xn1, 0);
        mma(f1a, f1b);
        interleave();
    };
    // fp32 rows (down) or bf16 h / fp32 partials (gate/up) of a finished block, straight from the accumulators:
    // lane holds features 4 kg .. 4 kg + 3 of weight block i for token 16 wn + rl
    auto finish = [&](const TileInfo& ti, int ntile, int ks, bool zero) {
        const int m = brow + rl;
        if (m >= ti.rows) return;
        const size_t row = (size_t)ti.off + ti.m0 + m;
        const f32x4 z4 = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (KIND == GemmKind::DownF32) {
            float* yout = DENSE && S > 1 ? a.part + (size_t)ks * a.part_rows * N
                                         : (ks == 0 ? static_cast<float*>(a.out)
                                                    : a.part + (size_t)(ks - 1) * a.part_rows * N);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int col = ntile * 256 + 64 * wm + 16 * i + 4 * kg;
                if (col >= N) continue;
                if (!DENSE && a.out_bf16) {
                    uint2 v;
                    v.x = pack_bf16x2(acc[i][0], acc[i][1]);
                    v.y = pack_bf16x2(acc[i][2], acc[i][3]);
                    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + row * N + col) = v;
                } else {
                    *reinterpret_cast<f32x4*>(yout + row * N + col) = acc[i];
                    if (zero) *reinterpret_cast<f32x4*>(a.part + row * N + col) = z4; // plane 1
                }
            }
        } else {
            static_assert(KIND == GemmKind::GateUp, "the streamed kernel computes gate/up and fp32 down GEMMs");
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int col = ntile * 128 + 32 * wm + 16 * i + 4 * kg;
                if (col >= N) continue;
                if (S > 1) {
                    float* prow = a.part + (size_t)ks * a.part_rows * 2 * N + row * 2 * N;
                    *reinterpret_cast<f32x4*>(prow + col) = acc[i];
                    *reinterpret_cast<f32x4*>(prow + N + col) = acc[i + 2];
                    if (zero) { // plane 1
                        float* zrow = a.part + (size_t)a.part_rows * 2 * N + row * 2 * N;
                        *reinterpret_cast<f32x4*>(zrow + col) = z4;
                        *reinterpret_cast<f32x4*>(zrow + N + col) = z4;
                    }
                } else {
                    const f32x4 g = acc[i], u = acc[i + 2];
                    uint2 v;
                    v.x = pack_bf16x2(swiglu(g[0], u[0]), swiglu(g[1], u[1]));
                    v.y = pack_bf16x2(swiglu(g[2], u[2]), swiglu(g[3], u[3]));
                    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + row * N + col) = v;
                }
            }
        }
    };

    Piece pc;
    if (!piece_at(cursor, pc)) return;
    Src cur = source(pc.ti, pc.ntile, pc.sb);
    // the first piece's ring: steps 0 to 3 (every piece has a multiple of 4 steps); the first barrier waits
    // for X0 and W0
    copy(cur, ws0, xs0, 0);
    copy(cur, ws1, xs1, 1);
    copy(cur, ws2, xs2, 2);
    copy(cur, ws3, xs3, 3);
    __builtin_amdgcn_s_waitcnt(0x0070 | VP); // vmcnt(15) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    read(f0a, f0b, ws0, xs0, 0);
    for (;;) {
        Piece pn;
        const bool has = piece_at(pc.next, pn);
        // this piece's steps 0 .. n - 5, copying its steps 4 .. n - 1
        for (int s = 0; s + 8 <= pc.n; s += 4) {
            dstep(ws0, xs0, ws1, xs1, cur, s + 4);
            dstep(ws1, xs1, ws2, xs2, cur, s + 5);
            dstep(ws2, xs2, ws3, xs3, cur, s + 6);
            dstep(ws3, xs3, ws0, xs0, cur, s + 7);
        }
        // its last four steps copy the next piece's steps 0 .. 3, or (last piece) repeat its own last step
        Src nxt = cur;
        int z = pc.n - 1, dz = 0;
        if (has) {
            nxt = source(pn.ti, pn.ntile, pn.sb);
            z = 0;
            dz = 1;
        }
        dstep(ws0, xs0, ws1, xs1, nxt, z);
        dstep(ws1, xs1, ws2, xs2, nxt, z + dz);
        dstep(ws2, xs2, ws3, xs3, nxt, z + 2 * dz);
        dstep(ws3, xs3, ws0, xs0, nxt, z + 3 * dz);
        // the first-half fragments of the next piece's step 0 are in f0a / f0b now
        finish(pc.ti, pc.ntile, pc.plane, pc.zero);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (!has) break;
        pc = pn;
        cur = nxt;
    }
    __builtin_amdgcn_s_waitcnt(0x0070); // no copy into LDS may outlive the workgroup
}

template <GemmKind KIND, bool DENSE>
__global__ __launch_bounds__(kDThreads) void gemm_dma_stream_kernel(GemmArgs a, int ntn) {
    // 153 KB: four weight buffers of [256][64] bf16, four token buffers of [32][64], the staged tile list and
    // gather map
    __shared__ __attribute__((aligned(16))) uint16_t ws0[kDRows * kBK];
    __shared__ __attribute__((aligned(16))) uint16_t ws1[kDRows * kBK];
    __shared__ __attribute__((aligned(16))) uint16_t ws2[kDRows * kBK];
    __shared__ __attribute__((aligned(16))) uint16_t ws3[kDRows * kBK];
    __shared__ __attribute__((aligned(16))) uint16_t xs0[32 * kBK];
    __shared__ __attribute__((aligned(16))) uint16_t xs1[32 * kBK];
    __shared__ __attribute__((aligned(16))) uint16_t xs2[32 * kBK];
    __shared__ __attribute__((aligned(16))) uint16_t xs3[32 * kBK];
    __shared__ __attribute__((aligned(16))) int tl[4 * kStreamMaxTiles]; // tile-list entries, 4 ints each
    __shared__ int rt[kStreamMaxRows];
    dma_stream<KIND, DENSE>(a, ntn, ws0, ws1, ws2, ws3, xs0, xs1, xs2, xs3, tl, rt);
}

// Persistent form of the grouped DMA GEMM: one workgroup per CU takes blocks from its XCD's counter (then
// from the other XCDs') until none is left; each tile runs as in the one-shot kernel.
template <GemmKind KIND>
__global__ __launch_bounds__(kDThreads) void gemm_dma_persistent_kernel(GemmArgs a, int ntn) {
    __shared__ __attribute__((aligned(16))) uint16_t ws0[kDRows * kBK];
    __shared__ __attribute__((aligned(16))) uint16_t ws1[kDRows * kBK];
    __shared__ __attribute__((aligned(16))) uint16_t ws2[kDRows * kBK];
    __shared__ __attribute__((aligned(16))) uint16_t xs0[kDRows * kBK];
    __shared__ __attribute__((aligned(16))) uint16_t xs1[kDRows * kBK];
    int* mbox = reinterpret_cast<int*>(ws2); // thread 0 hands the next block to everyone through LDS
    const int x = (int)(blockIdx.x % kXcds);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int got = 0; // wave 0: the block claimed next
    if (wave == 0) {
        int g = -1;
        if (threadIdx.x == 0) g = grab_block(a, ntn, x);
        got = __builtin_amdgcn_readfirstlane(g);
    }
    for (;;) {
        if (wave == 0 && __builtin_amdgcn_mbcnt_lo(~0u, 0u) == 0) mbox[0] = got;
        __syncthreads();
        const int L = __builtin_amdgcn_readfirstlane(mbox[0]);
        __syncthreads(); // read by everyone before the next tile's copies land in ws2
        int ntile;
        TileInfo ti;
        if (L < 0 || !block_at<kDRows>(a, ntn, L, ti, ntile)) return;
        const int nb = (ti.rows + 31) >> 5;
#define MOE_DMA_TILE(NBV) dma_tile<KIND, false, NBV, true>(a, ti, ntile, ws0, ws1, ws2, xs0, xs1, wave, ntn, got)
        switch (nb) {
        case 1: MOE_DMA_TILE(1); break;
        case 2: MOE_DMA_TILE(2); break;
        case 3: MOE_DMA_TILE(3); break;
        case 4: MOE_DMA_TILE(4); break;
        case 5: MOE_DMA_TILE(5); break;
        case 6: MOE_DMA_TILE(6); break;
        case 7: MOE_DMA_TILE(7); break;
        default: MOE_DMA_TILE(8); break;
        }
#undef MOE_DMA_TILE
        // gate/up: a wave may still read the last K step's buffers (ws2 among them) when thread 0 writes the
        // mailbox (the down GEMM's epilogue starts with a barrier after the K loop and stages in ws0 / ws1)
        if (KIND == GemmKind::GateUp) __syncthreads();
    }
}

// ------------------------------------------------------------------------------------------------
// skinny kernel

constexpr int kSBM = kSkinnyBM; // tokens per tile
static_assert(kSBM == 16, "skinny tiling assumes one 16-token MFMA column block");
constexpr int kSU = 1;          // 64-wide K chunks per pipeline stage (K is a multiple of 64)

template <GemmKind KIND, bool DENSE>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(GemmArgs a, int ntn, int64_t tiles_per_split) {
    int64_t bid = blockIdx.x;
    // dense GEMMs with few workgroups split K: split s covers 64-wide chunks [s C / S, (s + 1) C / S) and
    // writes fp32 partials (gate/up: g and u side by side) for a reduction kernel
    int split = 0;
    const bool partials = DENSE && a.ksplit > 1;
    if (partials) {
        split = (int)(bid / (tiles_per_split * ntn));
        bid -= (int64_t)split * tiles_per_split * ntn;
    }
    const int ntile = (int)(bid % ntn);
    TileInfo ti;
    if (!tile_info<DENSE, kSBM>(a, bid / ntn, ti)) return;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int rl = lane & 15, kg = lane >> 4;
    const int K = a.K, N = a.N;

    const uint16_t* wsrc[2];
    int col0;
    if (KIND == GemmKind::GateUp) {
        col0 = ntile * 64 + wave * 16;
        wsrc[0] = weight_row(a.w_a, a.ws_a, ti, N, col0 + rl, K) + kg * 16;
        wsrc[1] = weight_row(a.w_b, a.ws_b, ti, N, col0 + rl, K) + kg * 16;
    } else {
        col0 = ntile * 128 + wave * 32;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            int n = col0 + b * 16 + rl;
            n = n < N ? n : N - 1;
            wsrc[b] = weight_row(a.w_a, a.ws_a, ti, N, n, K) + kg * 16;
        }
    }
    const uint16_t* xsrc = act_row<KIND, DENSE>(a, ti, rl) + kg * 16;

    // Two register stages: the loads of K chunk st + 2 are issued right after chunk st's MFMAs, so every
    // wave keeps two chunks of weights in flight while it computes (loads past the end re-read the last
    // chunk: in bounds, unused).
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    struct Stage {
        Pack16 w[kSU][2][2], x[kSU][2];
    };
    const int C = K / (64 * kSU);
    const int cb = partials ? (int)((int64_t)split * C / a.ksplit) : 0;
    const int nst = partials ? (int)((int64_t)(split + 1) * C / a.ksplit) - cb : C;
    auto load = [&](Stage& s, int st) {
        st = st < nst ? st : nst - 1;
        const int kk = (cb + st) * 64 * kSU;
#pragma unroll
        for (int u = 0; u < kSU; ++u) {
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                s.w[u][b][0] = load16(wsrc[b] + kk + u * 64);
                s.w[u][b][1] = load16(wsrc[b] + kk + u * 64 + 8);
            }
            s.x[u][0] = load16(xsrc + kk + u * 64);
            s.x[u][1] = load16(xsrc + kk + u * 64 + 8);
        }
    };
    auto compute = [&](const Stage& s) {
#pragma unroll
        for (int u = 0; u < kSU; ++u)
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                acc[b] = mfma16x16x32(s.w[u][b][0], s.x[u][0], acc[b]);
                acc[b] = mfma16x16x32(s.w[u][b][1], s.x[u][1], acc[b]);
            }
    };
    Stage s0, s1;
    load(s0, 0);
    load(s1, 1);
    int st = 0;
    for (; st + 2 <= nst; st += 2) {
        compute(s0);
        load(s0, st + 2);
        compute(s1);
        load(s1, st + 3);
    }
    if (st < nst) compute(s0);

    if (rl >= ti.rows) return;
    const size_t row = (size_t)ti.off + ti.m0 + rl;
    if (partials) {
        float* base = static_cast<float*>(a.out) + (size_t)split * a.dense_rows * (KIND == GemmKind::GateUp ? 2 * N : N);
        if (KIND == GemmKind::GateUp) {
            const int col = col0 + 4 * kg;
            float* o = base + row * 2 * N;
            *reinterpret_cast<float4*>(o + col) = make_float4(acc[0][0], acc[0][1], acc[0][2], acc[0][3]);
            *reinterpret_cast<float4*>(o + N + col) = make_float4(acc[1][0], acc[1][1], acc[1][2], acc[1][3]);
        } else {
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int col = col0 + b * 16 + 4 * kg;
                if (col >= N) continue;
                *reinterpret_cast<float4*>(base + row * N + col) = make_float4(acc[b][0], acc[b][1], acc[b][2], acc[b][3]);
            }
        }
        return;
    }
    if (KIND == GemmKind::GateUp) {
        const int col = col0 + 4 * kg;
        uint2 v;
        v.x = pack_bf16x2(swiglu(acc[0][0], acc[1][0]), swiglu(acc[0][1], acc[1][1]));
        v.y = pack_bf16x2(swiglu(acc[0][2], acc[1][2]), swiglu(acc[0][3], acc[1][3]));
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + row * N + col) = v;
    } else {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int col = col0 + b * 16 + 4 * kg;
            if (col >= N) continue;
            const f32x4 y = acc[b];
            if (KIND == GemmKind::DownF32 && !DENSE && a.out_bf16) { // per-slot rows as bf16
                uint2 v;
                v.x = pack_bf16x2(y[0], y[1]);
                v.y = pack_bf16x2(y[2], y[3]);
                *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + row * N + col) = v;
                continue;
            }
            *reinterpret_cast<float4*>(static_cast<float*>(a.out) + row * N + col) = make_float4(y[0], y[1], y[2], y[3]);
        }
    }
}

// Reductions of the split-K partials, in split order: gate/up -> h = bf16(silu(g) * u); down -> fp32 out.
__global__ __launch_bounds__(256) void reduce_swiglu_kernel(const float* __restrict__ part, int S, int rows, int N,
                                                            uint16_t* __restrict__ h) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; // 4 consecutive columns of one row
    if (i >= (int64_t)rows * N) return;
    const int64_t row = i / N, col = i % N;
    float g[4] = {0.f, 0.f, 0.f, 0.f}, u[4] = {0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < S; ++sp) {
        const float* p = part + ((size_t)sp * rows + row) * 2 * N + col;
        const float4 gv = *reinterpret_cast<const float4*>(p);
        const float4 uv = *reinterpret_cast<const float4*>(p + N);
        g[0] += gv.x; g[1] += gv.y; g[2] += gv.z; g[3] += gv.w;
        u[0] += uv.x; u[1] += uv.y; u[2] += uv.z; u[3] += uv.w;
    }
    uint2 v;
    v.x = pack_bf16x2(swiglu(g[0], u[0]), swiglu(g[1], u[1]));
    v.y = pack_bf16x2(swiglu(g[2], u[2]), swiglu(g[3], u[3]));
    *reinterpret_cast<uint2*>(h + row * N + col) = v;
}

// The same for a grouped gate/up launch whose K split the permutation chose: nothing to do when it is 1 (the
// GEMM wrote h itself).
__global__ __launch_bounds__(256) void reduce_swiglu_ksplit_kernel(const float* __restrict__ part,
                                                                   const int32_t* __restrict__ ksplit, int rows,
                                                                   int N, uint16_t* __restrict__ h) {
    const int S = ksplit[0];
    if (S < 2 || S > kMaxGateUpSplits) return;
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= (int64_t)rows * N) return;
    const int64_t row = i / N, col = i % N;
    float g[4] = {0.f, 0.f, 0.f, 0.f}, u[4] = {0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < S; ++sp) { // the K ranges in order
        const float* p = part + ((size_t)sp * rows + row) * 2 * N + col;
        const float4 gv = *reinterpret_cast<const float4*>(p), uv = *reinterpret_cast<const float4*>(p + N);
        g[0] += gv.x; g[1] += gv.y; g[2] += gv.z; g[3] += gv.w;
        u[0] += uv.x; u[1] += uv.y; u[2] += uv.z; u[3] += uv.w;
    }
    uint2 v;
    v.x = pack_bf16x2(swiglu(g[0], u[0]), swiglu(g[1], u[1]));
    v.y = pack_bf16x2(swiglu(g[2], u[2]), swiglu(g[3], u[3]));
    *reinterpret_cast<uint2*>(h + row * N + col) = v;
}


__global__ __launch_bounds__(256) void reduce_sum_kernel(const float* __restrict__ part, int S, int64_t n,
                                                         float* __restrict__ out) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= n) return;
    float4 acc = *reinterpret_cast<const float4*>(part + i);
    for (int sp = 1; sp < S; ++sp) {
        const float4 v = *reinterpret_cast<const float4*>(part + (size_t)sp * n + i);
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
    }
    *reinterpret_cast<float4*>(out + i) = acc;
}

// Compute units of the current device, asked once per device.
hipError_t cu_count(int& cus) {
    static std::atomic<int> cache[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64 && (cus = cache[dev].load(std::memory_order_relaxed)) > 0) return hipSuccess;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (cus <= 0) return hipErrorInvalidDevice;
    if (dev >= 0 && dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
    return hipSuccess;
}

// Every split S in `allow` (bit S) cuts nk K steps into ranges of a whole number of deep-ring periods.
bool ring_periods(int nk, int allow) {
    for (int S = 1; S <= kMaxDownSplits; ++S)
        if (((allow >> S) & 1) && (nk % S != 0 || (nk / S) % 4 != 0)) return false;
    return true;
}

template <GemmKind KIND, bool DENSE>
hipError_t launch_one(GemmPath path, const GemmArgs& a, int64_t grid_tiles, hipStream_t stream) {
    // bf16 output rows: grouped down GEMMs only, whole 64-column chunks, no K split
    if (a.out_bf16 && (KIND != GemmKind::DownF32 || DENSE || a.N % 64 != 0 || a.ksplit_dev != nullptr))
        return hipErrorInvalidValue;
    // the deep-ring kernel takes tiles of at most 32 rows: dense GEMMs of up to 32 rows, grouped ones whose
    // groups hold at most 32 rows (the caller's guarantee: no more than 32 tokens)
    if (a.deep && (path != GemmPath::Dma || (DENSE && a.dense_rows > 32) || a.work_ctr != nullptr))
        return hipErrorInvalidValue;
    // separate fp32 rows of a folded shared expert: the LDS-copy kernel's grouped down GEMM only
    if (a.out_shared != nullptr && (KIND != GemmKind::DownF32 || DENSE || path != GemmPath::Dma ||
                                    a.shared_rows <= 0 || a.ksplit_dev != nullptr))
        return hipErrorInvalidValue;
    const bool wide = path != GemmPath::Skinny;
    int ntn;
    if (wide)
        ntn = KIND == GemmKind::GateUp ? (a.N + kWBN / 2 - 1) / (kWBN / 2) : (a.N + kWBN - 1) / kWBN;
    else
        ntn = KIND == GemmKind::GateUp ? a.N / 64 : (a.N + 127) / 128;
    const int splits =
        (KIND == GemmKind::Logits || (DENSE && (path == GemmPath::Skinny || path == GemmPath::Dma))) && a.ksplit > 1
            ? a.ksplit : 1;
    // a dense split on the LDS-copy kernel writes fp32 partials of dense_rows rows per K range
    if constexpr (DENSE && KIND != GemmKind::Logits)
        if (path == GemmPath::Dma && splits > 1 && (a.part == nullptr || a.part_rows < a.dense_rows ||
                                                    a.K / kBK < splits))
            return hipErrorInvalidValue;
    int64_t blocks = grid_tiles * ntn * splits;
    if (blocks <= 0) return hipSuccess;
    // the largest K split the permutation may choose (bit S of ks_allow), each range at least one K step
    int smax = 1;
    if (KIND != GemmKind::Logits && !DENSE && path == GemmPath::Dma && a.ksplit_dev != nullptr) {
        for (int S = 2; S <= kMaxDownSplits; ++S)
            if ((a.ks_allow >> S) & 1) smax = S;
        if ((a.ks_allow >> (kMaxDownSplits + 1)) != 0 || (KIND == GemmKind::GateUp && smax > kMaxGateUpSplits))
            return hipErrorInvalidValue;
        if (a.part == nullptr || a.part_rows <= 0 || a.K < smax * kBK) return hipErrorInvalidValue;
        blocks *= smax; // room for the largest split
    }
    if (wide && !DENSE) blocks = (blocks + kXcds - 1) / kXcds * kXcds;
    if (path == GemmPath::Dma && !DENSE && a.xcd_bounds != nullptr) {
        if (ntn != dma_ntn(KIND == GemmKind::GateUp, a.N)) return hipErrorInvalidValue;
        blocks = kXcds * dma_xcd_cap(grid_tiles, ntn);
    }
    if constexpr (KIND != GemmKind::Logits && !DENSE) {
        if (path == GemmPath::Dma && a.work_ctr != nullptr) {
            // persistent: one workgroup per CU (fewer when there are fewer blocks)
            int cus = 0;
            const hipError_t e = cu_count(cus);
            if (e != hipSuccess) return e;
            int64_t g = (int64_t)cus < blocks ? cus : blocks;
            g = (g + kXcds - 1) / kXcds * kXcds;
            gemm_dma_persistent_kernel<KIND><<<dim3((unsigned)g), kDThreads, 0, stream>>>(a, ntn);
            return hipGetLastError();
        }
    }
    if constexpr (KIND != GemmKind::Logits) {
        // the streamed deep-ring kernel: the one-shot order, one workgroup per CU (a multiple of kXcds, so each
        // workgroup's blocks stay on one XCD's range of the order), blocks of a multiple of 4 K steps, the tile
        // list and gather map within its LDS staging
        const int nk = a.K / kBK;
        bool streamed = path == GemmPath::Dma && a.deep == 2 && a.xcd_bounds == nullptr && a.out_shared == nullptr;
        if (DENSE)
            streamed = streamed && splits >= 1 && nk % splits == 0 && (nk / splits) % 4 == 0;
        else
            streamed = streamed && ring_periods(nk, a.ksplit_dev != nullptr ? a.ks_allow | 2 : 2) &&
                       grid_tiles <= kStreamMaxTiles &&
                     (KIND != GemmKind::GateUp ||
                      (a.row_token != nullptr && a.rt_rows > 0 && a.rt_rows <= kStreamMaxRows));
        if (streamed) {
            int cus = 0;
            const hipError_t e = cu_count(cus);
            if (e != hipSuccess) return e;
            int64_t g = (int64_t)cus < blocks ? cus : blocks;
            g = (g + kXcds - 1) / kXcds * kXcds;
            gemm_dma_stream_kernel<KIND, DENSE><<<dim3((unsigned)g), kDThreads, 0, stream>>>(a, ntn);
            return hipGetLastError();
        }
    }
    if (blocks > 0xFFFFFFFFLL) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)blocks);
    if constexpr (KIND == GemmKind::Logits) {
        if (path != GemmPath::Wide) return hipErrorInvalidValue;
        gemm_wide_kernel<KIND, DENSE, kWideBM><<<grid, kWThreads, 0, stream>>>(a, ntn, grid_tiles);
    } else {
        if (path == GemmPath::Dma && a.deep)
            gemm_dma_deep_kernel<KIND, DENSE><<<grid, kDThreads, 0, stream>>>(a, ntn);
        else if (path == GemmPath::Dma)
            gemm_dma_kernel<KIND, DENSE><<<grid, kDThreads, 0, stream>>>(a, ntn);
        else if (path == GemmPath::Wide)
            gemm_wide_kernel<KIND, DENSE, kWideBM><<<grid, kWThreads, 0, stream>>>(a, ntn, grid_tiles);
        else if (path == GemmPath::Tall)
            gemm_wide_kernel<KIND, DENSE, kTallBM><<<grid, kWThreads, 0, stream>>>(a, ntn, grid_tiles);
        else
            gemm_skinny_kernel<KIND, DENSE><<<grid, 256, 0, stream>>>(a, ntn, grid_tiles);
    }
    return hipGetLastError();
}

} // namespace

hipError_t launch_reduce(GemmKind kind, const float* partial, int S, int rows, int N, void* out, hipStream_t stream) {
    const int64_t n = (int64_t)rows * N;
    if (n <= 0) return hipSuccess;
    const unsigned blocks = (unsigned)((n / 4 + 255) / 256);
    if (kind == GemmKind::GateUp)
        reduce_swiglu_kernel<<<blocks, 256, 0, stream>>>(partial, S, rows, N, static_cast<uint16_t*>(out));
    else
        reduce_sum_kernel<<<blocks, 256, 0, stream>>>(partial, S, n, static_cast<float*>(out));
    return hipGetLastError();
}

hipError_t launch_reduce_ksplit(const float* partial, const int32_t* ksplit, int rows, int N, uint16_t* h,
                                hipStream_t stream) {
    const int64_t n = (int64_t)rows * N;
    if (n <= 0) return hipSuccess;
    reduce_swiglu_ksplit_kernel<<<(unsigned)((n / 4 + 255) / 256), 256, 0, stream>>>(partial, ksplit, rows, N, h);
    return hipGetLastError();
}

hipError_t device_cus(int& cus) { return cu_count(cus); }

hipError_t launch_gemm(GemmKind kind, GemmPath path, const GemmArgs& a, int64_t grid_tiles, hipStream_t stream) {
    const bool dense = a.counts == nullptr;
    switch (kind) {
    case GemmKind::GateUp:
        return dense ? launch_one<GemmKind::GateUp, true>(path, a, grid_tiles, stream)
                     : launch_one<GemmKind::GateUp, false>(path, a, grid_tiles, stream);
    case GemmKind::DownF32:
        return dense ? launch_one<GemmKind::DownF32, true>(path, a, grid_tiles, stream)
                     : launch_one<GemmKind::DownF32, false>(path, a, grid_tiles, stream);
    case GemmKind::Logits:
        return dense ? launch_one<GemmKind::Logits, true>(path, a, grid_tiles, stream) : hipErrorInvalidValue;
    }
    return hipErrorInvalidValue;
}

} // namespace moe
