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
//  * wide   : 128 tokens x 128 weight rows per workgroup, K in steps of 64 staged through LDS (double
//             buffered, 16-byte chunks XOR-swizzled by row so MFMA fragment reads are conflict-free);
//             4 waves in a 2 x 2 grid, each 64 weight rows x 64 tokens (16 MFMA tiles).
//  * skinny : 16 tokens per tile for experts with few rows (decode). No LDS: each wave streams its own
//             weight rows straight from HBM with 32-byte loads per lane, several 64-wide K chunks in
//             flight, so the kernel runs at the weight-streaming bound.
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
};

template <bool DENSE, int BM>
__device__ __forceinline__ bool tile_info(const GemmArgs& a, int64_t mtile, TileInfo& ti) {
    if (DENSE) {
        ti.g = 0;
        ti.m0 = (int)(mtile * BM);
        ti.off = 0;
        ti.rows = min(BM, a.dense_rows - ti.m0);
        return ti.rows > 0;
    }
    if (mtile >= a.ntiles[0]) return false;
    const int2 t = a.tiles[mtile];
    if (t.x < 0 || t.x >= a.groups || t.y < 0) return false;
    ti.g = t.x;
    ti.m0 = t.y;
    ti.off = a.offsets[t.x];
    ti.rows = min(BM, a.counts[t.x] - t.y);
    return ti.rows > 0;
}

// Activation row for tile row m (clamped to the tile's last valid row: padded columns of the MFMA tile
// read a real row and are never stored).
template <GemmKind KIND, bool DENSE>
__device__ __forceinline__ const uint16_t* act_row(const GemmArgs& a, const TileInfo& ti, int m) {
    m = m < ti.rows ? m : ti.rows - 1;
    const int r = ti.off + ti.m0 + m;
    if (KIND == GemmKind::GateUp && !DENSE) return a.act + (size_t)a.row_token[r] * a.K;
    return a.act + (size_t)r * a.K;
}

// ------------------------------------------------------------------------------------------------
// wide kernel

constexpr int kWBM = kWideBM;   // tokens per tile
constexpr int kWBN = 128;       // weight rows per tile
static_assert(kWBM == 128, "wide tiling assumes 128 tokens");

// LDS tile: [128 rows][64 k] bf16; chunk c (8 bf16) of row r lives at chunk c ^ (r & 7).
__device__ __forceinline__ int lds_off(int row, int chunk) { return row * kBK + ((chunk ^ (row & 7)) << 3); }

template <GemmKind KIND, bool DENSE>
__global__ __launch_bounds__(256) void gemm_wide_kernel(GemmArgs a, int ntn) {
    const int64_t bid = blockIdx.x;
    const int ntile = (int)(bid % ntn);
    TileInfo ti;
    if (!tile_info<DENSE, kWBM>(a, bid / ntn, ti)) return;

    __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][kWBN * kBK];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wn = wave & 1, wm = wave >> 1;
    const int rl = lane & 15, kg = lane >> 4;
    const int K = a.K, N = a.N;

    // global -> LDS assignment: chunk c of rows r_i = (tid >> 3) + 32 i
    const int lc = tid & 7;
    const uint16_t* wsrc[4];
    const uint16_t* xsrc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = (tid >> 3) + 32 * i;
        if (KIND == GemmKind::GateUp) {
            const int slab = r >> 6, q = r & 63;
            const int n = ntile * 64 + slab * 32 + (q & 31);
            const uint16_t* base = q < 32 ? a.w_a : a.w_b;
            wsrc[i] = base + ((size_t)ti.g * N + n) * K + lc * 8;
        } else {
            int n = ntile * kWBN + r;
            n = n < N ? n : N - 1;
            wsrc[i] = a.w_a + ((size_t)ti.g * N + n) * K + lc * 8;
        }
        xsrc[i] = act_row<KIND, DENSE>(a, ti, r) + lc * 8;
    }

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    Pack16 wv[4], xv[4];
    auto gload = [&](int kk) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            wv[i] = load16(wsrc[i] + kk);
            xv[i] = load16(xsrc[i] + kk);
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = (tid >> 3) + 32 * i;
            store16(&lds[buf][0][lds_off(r, lc)], wv[i]);
            store16(&lds[buf][1][lds_off(r, lc)], xv[i]);
        }
    };

    const int nk = K / kBK;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * kBK);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int chunk = ks * 4 + kg;
            Pack16 af[4], bf[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) af[i] = load16(&lds[cur][0][lds_off(wn * 64 + i * 16 + rl, chunk)]);
#pragma unroll
            for (int j = 0; j < 4; ++j) bf[j] = load16(&lds[cur][1][lds_off(wm * 64 + j * 16 + rl, chunk)]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(af[i], bf[j], acc[i][j]);
        }
        if (kt + 1 < nk) lstore(cur ^ 1);
        __syncthreads();
    }

    // epilogue: lane holds features 4 kg + r of weight block i and token rl of token block j
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int m = wm * 64 + j * 16 + rl;
        if (m >= ti.rows) continue;
        const size_t row = (size_t)ti.off + ti.m0 + m;
        if (KIND == GemmKind::GateUp) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int col = ntile * 64 + wn * 32 + i * 16 + 4 * kg;
                const f32x4 g = acc[i][j], u = acc[i + 2][j];
                uint2 v;
                v.x = pack_bf16x2(swiglu(g[0], u[0]), swiglu(g[1], u[1]));
                v.y = pack_bf16x2(swiglu(g[2], u[2]), swiglu(g[3], u[3]));
                *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + row * N + col) = v;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int col = ntile * kWBN + wn * 64 + i * 16 + 4 * kg;
                if (col >= N) continue;
                const f32x4 y = acc[i][j];
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
}

// ------------------------------------------------------------------------------------------------
// skinny kernel

constexpr int kSBM = kSkinnyBM; // tokens per tile
static_assert(kSBM == 16, "skinny tiling assumes one 16-token MFMA column block");
constexpr int kUnroll = 4;      // 64-wide K chunks in flight per lane

template <GemmKind KIND, bool DENSE>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(GemmArgs a, int ntn) {
    const int64_t bid = blockIdx.x;
    const int ntile = (int)(bid % ntn);
    TileInfo ti;
    if (!tile_info<DENSE, kSBM>(a, bid / ntn, ti)) return;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int rl = lane & 15, kg = lane >> 4;
    const int K = a.K, N = a.N;

    // two 16-row weight blocks per wave: gate/up -> W1 and W3 rows of the same 16 h columns;
    // down -> 32 consecutive W2 rows
    const uint16_t* wsrc[2];
    int col0;
    if (KIND == GemmKind::GateUp) {
        col0 = ntile * 64 + wave * 16;
        const size_t rowoff = ((size_t)ti.g * N + col0 + rl) * K + kg * 16;
        wsrc[0] = a.w_a + rowoff;
        wsrc[1] = a.w_b + rowoff;
    } else {
        col0 = ntile * 128 + wave * 32;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            int n = col0 + b * 16 + rl;
            n = n < N ? n : N - 1;
            wsrc[b] = a.w_a + ((size_t)ti.g * N + n) * K + kg * 16;
        }
    }
    const uint16_t* xsrc = act_row<KIND, DENSE>(a, ti, rl) + kg * 16;

    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    const int kfull = K / (64 * kUnroll) * (64 * kUnroll);
    for (int kk = 0; kk < kfull; kk += 64 * kUnroll) {
        Pack16 w[kUnroll][2][2], xr[kUnroll][2];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                w[u][b][0] = load16(wsrc[b] + kk + u * 64);
                w[u][b][1] = load16(wsrc[b] + kk + u * 64 + 8);
            }
            xr[u][0] = load16(xsrc + kk + u * 64);
            xr[u][1] = load16(xsrc + kk + u * 64 + 8);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                acc[b] = mfma16x16x32(w[u][b][0], xr[u][0], acc[b]);
                acc[b] = mfma16x16x32(w[u][b][1], xr[u][1], acc[b]);
            }
    }
    for (int kk = kfull; kk < K; kk += 64) {
        const Pack16 x0 = load16(xsrc + kk), x1 = load16(xsrc + kk + 8);
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            acc[b] = mfma16x16x32(load16(wsrc[b] + kk), x0, acc[b]);
            acc[b] = mfma16x16x32(load16(wsrc[b] + kk + 8), x1, acc[b]);
        }
    }

    if (rl >= ti.rows) return;
    const size_t row = (size_t)ti.off + ti.m0 + rl;
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

template <GemmKind KIND, bool DENSE>
hipError_t launch_one(bool wide, const GemmArgs& a, int64_t grid_tiles, hipStream_t stream) {
    const int ntn = KIND == GemmKind::GateUp ? a.N / 64 : (a.N + 127) / 128;
    const int64_t blocks = grid_tiles * ntn;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0xFFFFFFFFLL) return hipErrorInvalidConfiguration;
    if (wide)
        gemm_wide_kernel<KIND, DENSE><<<dim3((unsigned)blocks), 256, 0, stream>>>(a, ntn);
    else
        gemm_skinny_kernel<KIND, DENSE><<<dim3((unsigned)blocks), 256, 0, stream>>>(a, ntn);
    return hipGetLastError();
}

} // namespace

hipError_t launch_gemm(GemmKind kind, bool wide, const GemmArgs& a, int64_t grid_tiles, hipStream_t stream) {
    const bool dense = a.counts == nullptr;
    switch (kind) {
    case GemmKind::GateUp:
        return dense ? launch_one<GemmKind::GateUp, true>(wide, a, grid_tiles, stream)
                     : launch_one<GemmKind::GateUp, false>(wide, a, grid_tiles, stream);
    case GemmKind::Down:
        return dense ? launch_one<GemmKind::Down, true>(wide, a, grid_tiles, stream)
                     : launch_one<GemmKind::Down, false>(wide, a, grid_tiles, stream);
    case GemmKind::DownF32:
        return dense ? launch_one<GemmKind::DownF32, true>(wide, a, grid_tiles, stream)
                     : launch_one<GemmKind::DownF32, false>(wide, a, grid_tiles, stream);
    }
    return hipErrorInvalidValue;
}

} // namespace moe
