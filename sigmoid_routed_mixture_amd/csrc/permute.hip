// Permutation stage on gfx950: the T * k routing slots become expert-contiguous rows, ordered by token
// within each expert (a stable counting sort). Work is split in chunks of 256 tokens: each chunk builds
// an LDS bit matrix (expert x token-in-chunk), whose popcounts give the chunk's per-expert histogram and,
// below a token's bit, that token's rank inside the chunk. One workgroup then turns the histograms into
// per-expert offsets (an LDS prefix sum) and per-chunk bases, and lists the grouped-GEMM tiles
// ({expert | tile height << 16, first row}).
// Pages: the routed experts receive (hidden, indices, weights) (nnterp encyclopedia glm_moe_dsa, support():
// expert_indices and expert_weights are the experts' inputs); grouping rows by expert is how this build
// hands each expert its tokens.
#include "common.h"
#include "kernels.h"
#include "plan.h"

namespace moe {
namespace {

constexpr int kChunk = kPermChunk;
static_assert(kChunk == 256, "one thread per token of a chunk");

__device__ __forceinline__ void build_mask(uint32_t (*mask)[8], const int32_t* __restrict__ ids, int T, int E,
                                           int k) {
    const int tid = threadIdx.x;
    for (int i = tid; i < kMaxE * 8; i += 256) mask[i >> 3][i & 7] = 0u;
    __syncthreads();
    const int t = blockIdx.x * kChunk + tid;
    if (t < T) {
        for (int j = 0; j < k; ++j) {
            const int e = ids[(size_t)t * k + j];
            if (e >= 0 && e < E) atomicOr(&mask[e][tid >> 5], 1u << (tid & 31));
        }
    }
    __syncthreads();
}

__global__ __launch_bounds__(256) void perm_count_kernel(const int32_t* __restrict__ ids, int T, int E, int k,
                                                         int32_t* __restrict__ chunk_counts) {
    __shared__ uint32_t mask[kMaxE][8];
    build_mask(mask, ids, T, E, k);
    const int e = threadIdx.x;
    if (e < E) {
        int c = 0;
#pragma unroll
        for (int w = 0; w < 8; ++w) c += __popc(mask[e][w]);
        chunk_counts[(size_t)blockIdx.x * E + e] = c;
    }
}

// Exclusive prefix sum over the 256 threads of a workgroup.
__device__ __forceinline__ int block_exclusive_scan(int v, int* sh, int* total) {
    const int tid = threadIdx.x;
    sh[tid] = v;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
        const int a = tid >= off ? sh[tid - off] : 0;
        __syncthreads();
        sh[tid] += a;
        __syncthreads();
    }
    const int incl = sh[tid];
    *total = sh[255];
    __syncthreads();
    return incl - v;
}

// Appends the folded shared expert's tiles (group E, all shared_rows tokens, its rows from shared_off on)
// after the routed ones.
__device__ __forceinline__ int append_shared_tiles(int4* __restrict__ tiles, int32_t* __restrict__ ntiles,
                                                   int routed_tiles, int E, int shared_rows, int shared_off,
                                                   int BM) {
    const int tid = threadIdx.x;
    int ns = 0;
    if (shared_rows > 0) {
        const int hs = tile_height(shared_rows, BM);
        ns = (shared_rows + hs - 1) / hs;
        for (int i = tid; i < ns; i += 256)
            tiles[routed_tiles + i] = make_int4(E | (hs << 16), i * hs, shared_rows, shared_off);
    }
    if (tid == 0) ntiles[0] = routed_tiles + ns;
    return routed_tiles + ns;
}

// The K splits of a decode-sized launch's gate/up and down GEMMs (thread 0).
__device__ __forceinline__ void write_ksplit(const XcdSplit& sp, int all_tiles) {
    if (sp.ksplit != nullptr && threadIdx.x == 0)
        for (int i = 0; i < 2; ++i)
            sp.ksplit[i] =
                sp.ks_force > 0 ? sp.ks_force : decode_ksplit((int64_t)all_tiles * sp.ks_ntn[i], sp.cus);
}

// The work-balanced XCD split (plan.h) of the tile list just built, for both column-tile counts. Thread e
// holds expert e's row count n, tile height ht, tile count nt and first tile t0. Each boundary
// x * total / kXcds (in work units) falls inside one expert and is rounded down to one of its column
// tiles; thread 0 then clamps the boundaries so no XCD gets more than cap blocks.
__device__ void xcd_split(const XcdSplit& sp, int E, int n, int ht, int nt, int t0, int tiles_total, int* sh) {
    __shared__ int raw[2][kXcds + 1];
    __shared__ int totals[2];
    const int e = threadIdx.x;
    int c = 0; // work of one column of expert e's tiles
    if (e < E)
        for (int i = 0; i < nt; ++i) c += (min(ht, n - i * ht) + 31) / 32 + kDmaBlockCost;
    for (int v = 0; v < 2; ++v) {
        const int ntn = sp.ntn[v];
        int total = 0;
        const int w0 = block_exclusive_scan(e < E ? ntn * c : 0, sh, &total);
        if (e == 0) totals[v] = total;
        if (e < E && c > 0)
            for (int x = 1; x < kXcds; ++x) {
                const int B = (int)((int64_t)x * total / kXcds);
                if (B >= w0 && B < w0 + ntn * c) raw[v][x] = ntn * t0 + ((B - w0) / c) * nt;
            }
    }
    __syncthreads();
    if (e == 0)
        for (int v = 0; v < 2; ++v) {
            const int live = tiles_total * sp.ntn[v], cap = sp.cap[v];
            int32_t* b = sp.bounds + v * (kXcds + 1);
            int prev = 0;
            b[0] = 0;
            for (int x = 1; x < kXcds; ++x) {
                const int lo = max(prev, live - (kXcds - x) * cap), hi = min(prev + cap, live);
                const int r = totals[v] > 0 ? raw[v][x] : 0;
                prev = min(max(r, lo), hi);
                b[x] = prev;
            }
            b[kXcds] = live;
        }
}

__global__ __launch_bounds__(256) void perm_scan_kernel(int32_t* __restrict__ chunk_counts, int chunks, int E,
                                                        int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                        int4* __restrict__ tiles, int32_t* __restrict__ ntiles,
                                                        int BM, int shared_rows, int shared_off, XcdSplit split) {
    __shared__ int sh[256];
    const int e = threadIdx.x;
    int n = 0;
    if (e < E) {
        for (int c = 0; c < chunks; ++c) {
            int32_t* p = chunk_counts + (size_t)c * E + e;
            const int v = *p;
            *p = n; // in place: becomes the chunk's base row inside expert e
            n += v;
        }
        counts[e] = n;
    }
    int total = 0;
    const int off = block_exclusive_scan(e < E ? n : 0, sh, &total);
    if (e < E) offsets[e] = off;
    if (e == 0) offsets[E] = total;
    if (tiles == nullptr) return;
    const int ht = tile_height(n, BM);
    const int nt = (e < E && BM > 0) ? (n + ht - 1) / ht : 0;
    int tiles_total = 0;
    const int t0 = block_exclusive_scan(nt, sh, &tiles_total);
    for (int i = 0; i < nt; ++i) tiles[t0 + i] = make_int4(e | (ht << 16), i * ht, n, off);
    write_ksplit(split, append_shared_tiles(tiles, ntiles, tiles_total, E, shared_rows, shared_off, BM));
    if (split.bounds != nullptr) xcd_split(split, E, n, ht, nt, t0, tiles_total, sh);
    if (split.ctr != nullptr && e < 4 * kXcds) split.ctr[e] = 0;
}

__global__ __launch_bounds__(256) void perm_scatter_kernel(const int32_t* __restrict__ ids, int T, int E, int k,
                                                           const int32_t* __restrict__ offsets,
                                                           const int32_t* __restrict__ chunk_base,
                                                           int32_t* __restrict__ row_token,
                                                           int32_t* __restrict__ slot_row) {
    __shared__ uint32_t mask[kMaxE][8];
    build_mask(mask, ids, T, E, k);
    const int tid = threadIdx.x;
    const int t = blockIdx.x * kChunk + tid;
    if (t >= T) return;
    const int w = tid >> 5;
    const uint32_t below = (1u << (tid & 31)) - 1u;
    for (int j = 0; j < k; ++j) {
        const int e = ids[(size_t)t * k + j];
        if (e < 0 || e >= E) {
            slot_row[(size_t)t * k + j] = -1;
            continue;
        }
        int rank = __popc(mask[e][w] & below);
        for (int v = 0; v < w; ++v) rank += __popc(mask[e][v]);
        const int row = offsets[e] + chunk_base[(size_t)blockIdx.x * E + e] + rank;
        row_token[row] = t;
        slot_row[(size_t)t * k + j] = row;
    }
}

// The whole permutation in one workgroup when all tokens fit one chunk (decode): histogram, offsets and
// tile list, then the scatter, with the bit matrix kept in LDS between them.
__global__ __launch_bounds__(256) void perm_single_kernel(const int32_t* __restrict__ ids, int T, int E, int k,
                                                          int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                          int4* __restrict__ tiles, int32_t* __restrict__ ntiles,
                                                          int BM, int shared_rows, XcdSplit split,
                                                          int32_t* __restrict__ row_token,
                                                          int32_t* __restrict__ slot_row) {
    __shared__ uint32_t mask[kMaxE][8];
    __shared__ int sh[256];
    __shared__ int offs[kMaxE];
    build_mask(mask, ids, T, E, k);
    const int tid = threadIdx.x;
    int n = 0;
    if (tid < E) {
#pragma unroll
        for (int w = 0; w < 8; ++w) n += __popc(mask[tid][w]);
        counts[tid] = n;
    }
    int total = 0;
    const int off = block_exclusive_scan(tid < E ? n : 0, sh, &total);
    if (tid < E) {
        offsets[tid] = off;
        offs[tid] = off;
    }
    if (tid == 0) offsets[E] = total;
    if (tiles != nullptr) {
        const int ht = tile_height(n, BM);
        const int nt = (tid < E && BM > 0) ? (n + ht - 1) / ht : 0;
        int tiles_total = 0;
        const int t0 = block_exclusive_scan(nt, sh, &tiles_total);
        for (int i = 0; i < nt; ++i) tiles[t0 + i] = make_int4(tid | (ht << 16), i * ht, n, off);
        write_ksplit(split, append_shared_tiles(tiles, ntiles, tiles_total, E, shared_rows, T * k, BM));
        if (split.bounds != nullptr) xcd_split(split, E, n, ht, nt, t0, tiles_total, sh);
        if (split.ctr != nullptr && tid < 4 * kXcds) split.ctr[tid] = 0;
    }
    __syncthreads();
    const int t = tid;
    if (t >= T) return;
    const int w = tid >> 5;
    const uint32_t below = (1u << (tid & 31)) - 1u;
    for (int j = 0; j < k; ++j) {
        const int e = ids[(size_t)t * k + j];
        if (e < 0 || e >= E) {
            slot_row[(size_t)t * k + j] = -1;
            continue;
        }
        int rank = __popc(mask[e][w] & below);
        for (int v = 0; v < w; ++v) rank += __popc(mask[e][v]);
        const int row = offs[e] + rank;
        row_token[row] = t;
        slot_row[(size_t)t * k + j] = row;
    }
}

__global__ __launch_bounds__(256) void gather_rows_kernel(const uint16_t* __restrict__ x,
                                                          const int32_t* __restrict__ row_token,
                                                          const int32_t* __restrict__ offsets, int E, int T, int H,
                                                          uint16_t* __restrict__ x_perm) {
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= offsets[E]) return;
    const int t = row_token[r];
    if (t < 0 || t >= T) return;
    const int lane = threadIdx.x & 63;
    const uint16_t* src = x + (size_t)t * H;
    uint16_t* dst = x_perm + (size_t)r * H;
    for (int c = lane; c < H / 8; c += 64) store16(dst + c * 8, load16(src + c * 8));
}

__global__ void fill_i32_kernel(int32_t* __restrict__ p, int64_t n, int32_t v) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

} // namespace

hipError_t launch_permute(const int32_t* ids, int T, int E, int k, int32_t* counts, int32_t* offsets,
                          int32_t* row_token, int32_t* slot_row, int32_t* chunk_scratch, int4* tiles,
                          int32_t* ntiles, int BM, int shared_rows, const XcdSplit& split, hipStream_t stream) {
    const int chunks = (T + kChunk - 1) / kChunk;
    if (chunks == 1) {
        perm_single_kernel<<<1, 256, 0, stream>>>(ids, T, E, k, counts, offsets, tiles, ntiles, BM, shared_rows,
                                                  split, row_token, slot_row);
        return hipGetLastError();
    }
    perm_count_kernel<<<chunks, 256, 0, stream>>>(ids, T, E, k, chunk_scratch);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    perm_scan_kernel<<<1, 256, 0, stream>>>(chunk_scratch, chunks, E, counts, offsets, tiles, ntiles, BM,
                                            shared_rows, T * k, split);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    perm_scatter_kernel<<<chunks, 256, 0, stream>>>(ids, T, E, k, offsets, chunk_scratch, row_token, slot_row);
    return hipGetLastError();
}

hipError_t launch_gather_rows(const uint16_t* x, const int32_t* row_token, const int32_t* offsets, int E, int T,
                              int H, int rows_max, uint16_t* x_perm, hipStream_t stream) {
    gather_rows_kernel<<<(rows_max + 3) / 4, 256, 0, stream>>>(x, row_token, offsets, E, T, H, x_perm);
    return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    fill_i32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(p, n, v);
    return hipGetLastError();
}

} // namespace moe
