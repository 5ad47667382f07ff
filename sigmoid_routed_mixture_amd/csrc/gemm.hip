// Grouped GEMMs of the SwiGLU experts on gfx950 (bf16 MFMA 16x16x32, fp32 accumulation).
//
// Gate/up GEMM: for the rows of one expert, g = x W1^T and u = x W3^T for the same output columns in one
// workgroup, and the epilogue writes h = silu(g) * u as bf16. Down GEMM: y = h W2^T, written as bf16
// per-slot rows (routed) or fp32 (shared expert). Pages: open-model-atlas GLM-5 "MoE transformer block",
// "All 43 steps": g = x W1, u = x W3, a = g sigma(g), h = a * u, E_i = h W2, and the same four steps for
// the shared expert.
//
// Weights are the MFMA A operand (rows = output features) and tokens the B operand (columns), so a lane's
// four accumulator elements are four consecutive output features of one token row: 8-byte bf16 stores.
//
// Two kernels:
//  * wide   : 128 or 256 tokens x 256 weight rows per 8-wave workgroup. Each wave streams its own 32
//             weight rows from HBM into MFMA registers; the token tile goes through double-buffered LDS.
//             The 128-token form also computes the router logits (dense, K split across workgroups).
//  * skinny : 16 tokens per tile for experts with few rows (decode). No LDS: each wave streams its own
//             weight rows straight from HBM with 32-byte loads per lane, two 64-wide K chunks in flight
//             ahead of its MFMAs, so the kernel runs at the weight-streaming bound.
// Both take their (expert, first row) tiles from the device-side list the permutation builds; the grid is
// an upper bound and workgroups past the list's length exit at once.
#include "common.h"
#include "kernels.h"
#include "plan.h"

namespace moe {
namespace {

constexpr int kBK = 64;

struct TileInfo {
    int g, m0, rows, off;
    bool shared; // the folded shared expert (group index == groups)
};

// Row n of a group's weights: routed experts from w ([groups][N][K]), the folded shared expert from ws.
__device__ __forceinline__ const uint16_t* weight_row(const uint16_t* w, const uint16_t* ws, const TileInfo& ti,
                                                      int N, int n, int K) {
    return ti.shared ? ws + (size_t)n * K : w + ((size_t)ti.g * N + n) * K;
}

// Rows of group g: the routed counts, or all shared_rows tokens for the folded shared expert.
__device__ __forceinline__ int group_rows(const GemmArgs& a, int g) {
    return g < a.groups ? a.counts[g] : a.shared_rows;
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
    const int2 t = a.tiles[mtile];
    const int g = t.x & 0xFFFF, ht = t.x >> 16;
    const int ngroups = a.groups + (a.shared_rows > 0 ? 1 : 0);
    if (g >= ngroups || ht <= 0 || ht > BM || t.y < 0) return false;
    ti.g = g;
    ti.m0 = t.y;
    ti.shared = g == a.groups;
    ti.off = ti.shared ? a.shared_off : a.offsets[g];
    ti.rows = min(ht, group_rows(a, g) - t.y);
    return ti.rows > 0;
}

// Workgroup -> (token tile, output-column tile) of the grouped wide GEMM. The live blocks go in
// expert-major order and each XCD takes one contiguous eighth of it: the token tiles that share a slice
// of an expert's weights run side by side on one XCD, and so do the column tiles that share a token
// tile, so both come from HBM about once instead of once per XCD.
template <int BM>
__device__ __forceinline__ bool grouped_block(const GemmArgs& a, int ntn, int64_t bid, int64_t& mtile,
                                              int& ntile) {
    const int64_t L = xcd_block_order(bid, (int64_t)a.ntiles[0] * ntn);
    if (L < 0) return false;
    const int2 entry = a.tiles[L / ntn];
    const int g = entry.x & 0xFFFF, ht = entry.x >> 16;
    const int ngroups = a.groups + (a.shared_rows > 0 ? 1 : 0);
    if (g >= ngroups || ht <= 0 || ht > BM || entry.y < 0) return false;
    const int m = (group_rows(a, g) + ht - 1) / ht;
    if (m <= 0) return false;
    mtile = expert_major_tile(L, ntn, entry.y / ht, m, ntile);
    return true;
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
                if (KIND == GemmKind::Down) {
                    uint2 v;
                    v.x = pack_bf16x2(y[0], y[1]);
                    v.y = pack_bf16x2(y[2], y[3]);
                    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + row * N + col) = v;
                } else {
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
    int64_t mtile;
    if (DENSE) {
        ntile = (int)(bid % ntn);
        mtile = bid / ntn;
    } else if (!grouped_block<BM>(a, ntn, bid, mtile, ntile)) {
        return;
    }
    TileInfo ti;
    if (!tile_info<DENSE, BM>(a, mtile, ti)) return;

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
            if (KIND == GemmKind::Down) {
                uint2 v;
                v.x = pack_bf16x2(y[0], y[1]);
                v.y = pack_bf16x2(y[2], y[3]);
                *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + row * N + col) = v;
            } else {
                *reinterpret_cast<float4*>(static_cast<float*>(a.out) + row * N + col) =
                    make_float4(y[0], y[1], y[2], y[3]);
            }
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

template <GemmKind KIND, bool DENSE>
hipError_t launch_one(GemmPath path, const GemmArgs& a, int64_t grid_tiles, hipStream_t stream) {
    const bool wide = path != GemmPath::Skinny;
    int ntn;
    if (wide)
        ntn = KIND == GemmKind::GateUp ? (a.N + kWBN / 2 - 1) / (kWBN / 2) : (a.N + kWBN - 1) / kWBN;
    else
        ntn = KIND == GemmKind::GateUp ? a.N / 64 : (a.N + 127) / 128;
    const int splits = (KIND == GemmKind::Logits || (!wide && DENSE)) && a.ksplit > 1 ? a.ksplit : 1;
    int64_t blocks = grid_tiles * ntn * splits;
    if (blocks <= 0) return hipSuccess;
    if (wide && !DENSE) blocks = (blocks + kXcds - 1) / kXcds * kXcds;
    if (blocks > 0xFFFFFFFFLL) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)blocks);
    if constexpr (KIND == GemmKind::Logits) {
        if (path != GemmPath::Wide) return hipErrorInvalidValue;
        gemm_wide_kernel<KIND, DENSE, kWideBM><<<grid, kWThreads, 0, stream>>>(a, ntn, grid_tiles);
    } else {
        if (path == GemmPath::Wide)
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

hipError_t launch_gemm(GemmKind kind, GemmPath path, const GemmArgs& a, int64_t grid_tiles, hipStream_t stream) {
    const bool dense = a.counts == nullptr;
    switch (kind) {
    case GemmKind::GateUp:
        return dense ? launch_one<GemmKind::GateUp, true>(path, a, grid_tiles, stream)
                     : launch_one<GemmKind::GateUp, false>(path, a, grid_tiles, stream);
    case GemmKind::Down:
        return dense ? launch_one<GemmKind::Down, true>(path, a, grid_tiles, stream)
                     : launch_one<GemmKind::Down, false>(path, a, grid_tiles, stream);
    case GemmKind::DownF32:
        return dense ? launch_one<GemmKind::DownF32, true>(path, a, grid_tiles, stream)
                     : launch_one<GemmKind::DownF32, false>(path, a, grid_tiles, stream);
    case GemmKind::Logits:
        return dense ? launch_one<GemmKind::Logits, true>(path, a, grid_tiles, stream) : hipErrorInvalidValue;
    }
    return hipErrorInvalidValue;
}

} // namespace moe
