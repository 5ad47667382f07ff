// Permutation stage on gfx950: the T * k routing slots become expert-contiguous rows, ordered by token
// within each expert (a stable counting sort). Work is split in chunks of 256 tokens: each chunk builds
// an LDS bit matrix (expert x token-in-chunk), whose popcounts give the chunk's per-expert histogram and,
// below a token's bit, that token's rank inside the chunk. One workgroup then turns the histograms into
// per-expert offsets (an LDS prefix sum) and per-chunk bases, and lists the grouped-GEMM tiles (plan.h's
// tile words, in the plain or the dealt order).
// Pages: the routed experts receive (hidden, indices, weights) (nnterp encyclopedia glm_moe_dsa, support():
// expert_indices and expert_weights are the experts' inputs); grouping rows by expert is how this library
// hands each expert its tokens.
#include "common.h"
#include "kernels.h"
#include "plan.h"
#include "topk.h"

namespace moe {
namespace {

constexpr int kChunk = kPermChunk;
static_assert(kChunk == 256, "one thread per token of a chunk");

// Bit matrix of the chunk of tokens [t0, t0 + 256): bit (t - t0) of expert e's row is set when token t
// chose e.
__device__ __forceinline__ void build_mask(uint32_t (*mask)[8], const int32_t* __restrict__ ids, int T, int E,
                                           int k, int t0) {
    const int tid = threadIdx.x;
    for (int i = tid; i < kMaxE * 8; i += 256) mask[i >> 3][i & 7] = 0u;
    __syncthreads();
    const int t = t0 + tid;
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
    build_mask(mask, ids, T, E, k, blockIdx.x * kChunk);
    const int e = threadIdx.x;
    if (e < E) {
        int c = 0;
#pragma unroll
        for (int w = 0; w < 8; ++w) c += __popc(mask[e][w]);
        chunk_counts[(size_t)blockIdx.x * E + e] = c;
    }
}

// Exclusive prefix sum over the 256 threads of a workgroup: an inclusive scan within each wave by lane
// shuffles, the four wave totals through LDS (sh[0..3]), two barriers in all (the second lets the caller
// reuse sh at once).
__device__ __forceinline__ int block_exclusive_scan(int v, int* sh, int* total) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) sh[w] = x;
    __syncthreads();
    int before = 0;
#pragma unroll
    for (int i = 0; i < 3; ++i)
        if (i < w) before += sh[i];
    *total = sh[0] + sh[1] + sh[2] + sh[3];
    __syncthreads();
    return before + x - v;
}

// Writes tiles [f0, f0 + cnt) of group g (n rows, tiles of height ht, its rows from `off` on in the permuted
// buffers) at tiles[t0 ...] in the plain order: chunks of up to `cap` consecutive tiles.
__device__ __forceinline__ void write_plain_tiles(int4* __restrict__ tiles, int t0, int g, int n, int ht, int cnt,
                                                  int off, int cap, int f0 = 0) {
    const int nc = plain_chunks(cnt, cap);
    for (int c = 0; c < nc; ++c) {
        const int f = chunk_first(c, nc, cnt), cm = chunk_first(c + 1, nc, cnt) - f;
        for (int ci = 0; ci < cm; ++ci)
            tiles[t0 + f + ci] = make_int4(tile_word(g, ht, ci, cm), (f0 + f + ci) * ht, n, off);
    }
}

// The shared group (group E, shared_rows rows) cut into kXcds pieces, piece j holding its tiles
// [chunk_first(j, kXcds, ns), chunk_first(j + 1, kXcds, ns)), placed right before routed expert
// shared_piece_at(j, E): with equal-count XCD ranges over the list, each XCD's range then holds about one
// piece. Pieces before expert e's tiles: those with shared_piece_at(j, E) <= e.
__device__ __forceinline__ int shared_piece_at(int j, int E) { return (j * E + kXcds - 1) / kXcds; }
__device__ __forceinline__ int shared_pieces_before(int e, int E) {
    int J = 0;
    for (int j = 0; j < kXcds; ++j) J += shared_piece_at(j, E) <= e ? 1 : 0;
    return J;
}

// Appends the folded shared expert's tiles (group E, all shared_rows tokens, its rows from shared_off on)
// after the routed ones.
__device__ __forceinline__ int append_shared_tiles(int4* __restrict__ tiles, int32_t* __restrict__ ntiles,
                                                   int routed_tiles, int E, int shared_rows, int shared_off,
                                                   int BM, int cap) {
    const int tid = threadIdx.x;
    int ns = 0;
    if (shared_rows > 0) {
        const int hs = tile_height(shared_rows, BM);
        ns = (shared_rows + hs - 1) / hs;
        if (tid == 0) write_plain_tiles(tiles, routed_tiles, E, shared_rows, hs, ns, shared_off, cap);
    }
    if (tid == 0) ntiles[0] = routed_tiles + ns;
    return routed_tiles + ns;
}

// The dealt order of plan.h, built by the 256 threads of the scan workgroup: thread e holds routed expert
// e's row count n, tile height ht, tile count nt and first permuted row off (e < E); the folded shared
// expert (shared_rows > 0: group E, its rows from shared_off on) comes before every expert. Writes the tile
// list, its length and, for both GEMMs (ntn[v] column tiles), the XCD ranges of the blocks. Returns the
// number of tiles, or -1 (nothing written) when the chunks exceed kMaxDealtChunks.
__device__ int write_dealt_tiles(const XcdSplit& sp, int4* __restrict__ tiles, int32_t* __restrict__ ntiles, int E,
                                 int n, int ht, int nt, int off, int shared_rows, int shared_off, int BM, int* sh) {
    __shared__ int rows_of[kMaxE];
    __shared__ int by_rank[kMaxE];
    __shared__ int slots[kXcds * kDealtSlots];
    const int e = threadIdx.x;
    rows_of[e] = e < E ? n : 0;
    for (int i = e; i < kXcds * kDealtSlots; i += 256) slots[i] = 0;
    __syncthreads();
    // rank among the experts: rows descending, then index (a permutation of 0 .. 255, empty experts last),
    // or the index itself
    int rank = e;
    if (sp.dealt != kDealtIndex) {
        rank = 0;
        for (int j = 0; j < kMaxE; ++j) {
            const int nj = rows_of[j];
            rank += (nj > rows_of[e] || (nj == rows_of[e] && j < e)) ? 1 : 0;
        }
    }
    const int nc = e < E ? dealt_chunks(nt) : 0;
    const int hs = shared_rows > 0 ? tile_height(shared_rows, BM) : 0;
    const int ns = shared_rows > 0 ? (shared_rows + hs - 1) / hs : 0;
    const int ncs = dealt_chunks(ns);
    by_rank[rank] = nc;
    __syncthreads();
    int routed_chunks = 0;
    const int before = block_exclusive_scan(by_rank[e], sh, &routed_chunks); // chunks ahead of rank e
    __syncthreads();
    by_rank[e] = before;
    __syncthreads();
    const int all = ncs + routed_chunks;
    if (all > kMaxDealtChunks) return -1; // uniform: every thread sees the same totals
    const int c0 = ncs + by_rank[rank];  // this expert's first chunk in dealing order
    // the (XCD, slot) place of chunk c in the list
    auto place = [&](int c) {
        const int x = deal_xcd(c);
        const int sl = sp.dealt == kDealtAlternating ? alternate_slot(deal_slot(c), deal_count(x, all)) : deal_slot(c);
        return x * kDealtSlots + sl;
    };
    for (int c = 0; c < nc; ++c) slots[place(c0 + c)] = chunk_first(c + 1, nc, nt) - chunk_first(c, nc, nt);
    if (e == 0)
        for (int c = 0; c < ncs; ++c) slots[place(c)] = chunk_first(c + 1, ncs, ns) - chunk_first(c, ncs, ns);
    __syncthreads();
    // first tile of every (XCD, slot): an exclusive scan of the XCD-major slot array, 8 slots per thread
    constexpr int per = kXcds * kDealtSlots / 256;
    int part = 0;
    for (int i = 0; i < per; ++i) part += slots[e * per + i];
    int total = 0;
    int run = block_exclusive_scan(part, sh, &total);
    for (int i = 0; i < per; ++i) {
        const int v = slots[e * per + i];
        slots[e * per + i] = run;
        run += v;
    }
    __syncthreads();
    for (int c = 0; c < nc; ++c) {
        const int f = chunk_first(c, nc, nt), cm = chunk_first(c + 1, nc, nt) - f;
        const int t0 = slots[place(c0 + c)];
        for (int ci = 0; ci < cm; ++ci) tiles[t0 + ci] = make_int4(tile_word(e, ht, ci, cm), (f + ci) * ht, n, off);
    }
    if (e == 0)
        for (int c = 0; c < ncs; ++c) {
            const int f = chunk_first(c, ncs, ns), cm = chunk_first(c + 1, ncs, ns) - f;
            const int t0 = slots[place(c)];
            for (int ci = 0; ci < cm; ++ci)
                tiles[t0 + ci] = make_int4(tile_word(E, hs, ci, cm), (f + ci) * hs, shared_rows, shared_off);
        }
    if (e < 2 * (kXcds + 1)) {
        const int v = e / (kXcds + 1), x = e % (kXcds + 1);
        sp.bounds[e] = sp.ntn[v] * (x < kXcds ? slots[x * kDealtSlots] : total);
    }
    if (e == 0) ntiles[0] = total;
    return total;
}

// The K splits of a decode-sized launch's gate/up and down GEMMs (thread 0): decode_ksplit_gate_up and
// decode_ksplit_down among each GEMM's allowed splits, or forced: ks_force 2 splits in two where that is
// allowed, 3 takes the largest allowed split.
__device__ __forceinline__ void write_ksplit(const XcdSplit& sp, int all_tiles) {
    if (sp.ksplit != nullptr && threadIdx.x == 0)
        for (int i = 0; i < 2; ++i) {
            const int allow = sp.ks_allow[i] | 2;
            const int64_t b = (int64_t)all_tiles * sp.ks_ntn[i];
            int S = i == 0 ? ((allow >> 2) & 1 ? decode_ksplit_gate_up(b, sp.cus, (allow >> 4) & 1) : 1)
                           : decode_ksplit_down(b, sp.cus, allow);
            if (sp.ks_force > 0) {
                const int cap = sp.ks_force == 2 ? 2 : kMaxDownSplits;
                S = 1;
                for (int v = 2; v <= cap; ++v)
                    if ((allow >> v) & 1) S = v;
            }
            const int sk = sp.ks_force == 0 && sp.ks_streamk[i] && ((allow >> 2) & 1) && decode_streamk(b, sp.cus);
            sp.ksplit[i] = sk ? 2 : S;
            sp.ksplit[2 + i] = sk;
        }
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

// The grouped-GEMM tile list of every expert (thread e: expert e with n rows, its rows from `off` on) and
// of the folded shared expert, in the dealt order when asked and possible, else the plain order (experts in
// index order, the shared expert last); then the K splits, the plain order's work-balanced XCD split and the
// zeroed block counters.
__device__ void write_tiles(const XcdSplit& split, int4* __restrict__ tiles, int32_t* __restrict__ ntiles, int E,
                            int n, int off, int BM, int shared_rows, int shared_off, int* sh) {
    const int e = threadIdx.x;
    const int ht = tile_height(n, BM);
    const int nt = (e < E && BM > 0) ? (n + ht - 1) / ht : 0;
    int all_tiles = -1;
    if (split.dealt && split.bounds != nullptr)
        all_tiles = write_dealt_tiles(split, tiles, ntiles, E, n, ht, nt, off, shared_rows, shared_off, BM, sh);
    if (all_tiles < 0 && split.spread_shared && shared_rows > 0) {
        // plain order with the shared group's kXcds pieces spread through it
        __shared__ int routed_start[kMaxE + 1];
        const int cap = split.plain_cap > 0 ? split.plain_cap : kMaxChunkTiles;
        int routed_total = 0;
        const int t0r = block_exclusive_scan(nt, sh, &routed_total);
        routed_start[e] = t0r;
        if (e == 0) routed_start[kMaxE] = routed_total;
        __syncthreads();
        const int hs = tile_height(shared_rows, BM);
        const int ns = (shared_rows + hs - 1) / hs;
        if (nt > 0)
            write_plain_tiles(tiles, t0r + chunk_first(shared_pieces_before(e, E), kXcds, ns), e, n, ht, nt, off, cap);
        if (e < kXcds) {
            const int p = shared_piece_at(e, E); // p <= E: before expert p, or at the end
            const int f = chunk_first(e, kXcds, ns), cnt = chunk_first(e + 1, kXcds, ns) - f;
            const int at = (p < E ? routed_start[p] : routed_total) + f;
            if (cnt > 0) write_plain_tiles(tiles, at, E, shared_rows, hs, cnt, shared_off, cap, f);
        }
        all_tiles = routed_total + ns;
        if (e == 0) ntiles[0] = all_tiles;
        if (split.bounds != nullptr && e < 2 * (kXcds + 1)) { // equal block counts per XCD for both GEMMs
            const int v = e / (kXcds + 1), x = e % (kXcds + 1);
            const int live = all_tiles * split.ntn[v], chunk = (live + kXcds - 1) / kXcds;
            split.bounds[e] = min(x * chunk, live);
        }
    }
    if (all_tiles < 0) {
        const int cap = split.plain_cap > 0 ? split.plain_cap : kMaxChunkTiles;
        int tiles_total = 0;
        const int t0 = block_exclusive_scan(nt, sh, &tiles_total);
        if (nt > 0) write_plain_tiles(tiles, t0, e, n, ht, nt, off, cap);
        all_tiles = append_shared_tiles(tiles, ntiles, tiles_total, E, shared_rows, shared_off, BM, cap);
        if (split.bounds != nullptr) xcd_split(split, E, n, ht, nt, t0, tiles_total, sh);
    }
    write_ksplit(split, all_tiles);
    if (split.ctr != nullptr && e < 4 * kXcds) split.ctr[e] = 0;
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
    write_tiles(split, tiles, ntiles, E, n, off, BM, shared_rows, shared_off, sh);
}

__global__ __launch_bounds__(256) void perm_scatter_kernel(const int32_t* __restrict__ ids, int T, int E, int k,
                                                           const int32_t* __restrict__ offsets,
                                                           const int32_t* __restrict__ chunk_base,
                                                           int32_t* __restrict__ row_token,
                                                           int32_t* __restrict__ slot_row) {
    __shared__ uint32_t mask[kMaxE][8];
    build_mask(mask, ids, T, E, k, blockIdx.x * kChunk);
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
// tile list, then the scatter, with the bit matrix kept in LDS between them. Every thread of the 256-thread
// workgroup calls it (it holds barriers).
__device__ void permute_single(const int32_t* __restrict__ ids, int T, int E, int k, int32_t* __restrict__ counts,
                               int32_t* __restrict__ offsets, int4* __restrict__ tiles, int32_t* __restrict__ ntiles,
                               int BM, int shared_rows, const XcdSplit& split, int32_t* __restrict__ row_token,
                               int32_t* __restrict__ slot_row) {
    __shared__ uint32_t mask[kMaxE][8];
    __shared__ int sh[256];
    __shared__ int offs[kMaxE];
    build_mask(mask, ids, T, E, k, 0);
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
    if (tiles != nullptr) write_tiles(split, tiles, ntiles, E, n, off, BM, shared_rows, T * k, sh);
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

__global__ __launch_bounds__(256) void perm_single_kernel(const int32_t* __restrict__ ids, int T, int E, int k,
                                                          int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                          int4* __restrict__ tiles, int32_t* __restrict__ ntiles,
                                                          int BM, int shared_rows, XcdSplit split,
                                                          int32_t* __restrict__ row_token,
                                                          int32_t* __restrict__ slot_row) {
    permute_single(ids, T, E, k, counts, offsets, tiles, ntiles, BM, shared_rows, split, row_token, slot_row);
}

// Decode: the router's top-k and the permutation in one launch. Workgroup t sums token t's S partial logits
// in split order (one thread per expert, every load in flight at once) and one wave routes the token, as
// the router's few-token top-k kernel does. The wave then publishes the token's ids (an agent-scope fence
// before its ticket: the workgroups may run on different XCDs, each with its own L2) and takes a ticket;
// the workgroup that takes the last one (T - 1) fences again and runs the single-chunk permutation over
// every token's ids. The logits kernel zeroed the ticket, so exactly one workgroup permutes.
__global__ __launch_bounds__(256) void route_permute_few_kernel(
    const float* __restrict__ partial, int S, const float* __restrict__ bias, int T, int E, int k, float scale,
    int32_t* __restrict__ ids, float* __restrict__ gates, float* __restrict__ logits, int32_t* __restrict__ ticket,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int4* __restrict__ tiles,
    int32_t* __restrict__ ntiles, int BM, int shared_rows, XcdSplit split, int32_t* __restrict__ row_token,
    int32_t* __restrict__ slot_row) {
    __shared__ float zs[kMaxE];
    __shared__ int last;
    const int t = blockIdx.x;
    const int e = threadIdx.x;
    if (e < E) {
        const size_t stride = (size_t)T * E;
        const float* p = partial + (size_t)t * E + e;
        float v[kRouterMaxSplits];
#pragma unroll
        for (int i = 0; i < kRouterMaxSplits; ++i)
            if (i < S) v[i] = p[(size_t)i * stride];
        float z = 0.f;
#pragma unroll
        for (int i = 0; i < kRouterMaxSplits; ++i)
            if (i < S) z += v[i];
        zs[e] = z;
    }
    __syncthreads();
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        float z4[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) z4[q] = lane + 64 * q < E ? zs[lane + 64 * q] : 0.f;
        topk_token(z4, t, E, k, scale, bias, ids, gates, logits);
        __threadfence(); // this token's ids reach every XCD before its ticket
        if (lane == 0) last = atomicAdd(ticket, 1) == T - 1 ? 1 : 0;
    }
    __syncthreads();
    if (!last) return; // uniform over the workgroup
    __threadfence();   // every token's ids, as published before their tickets
    permute_single(ids, T, E, k, counts, offsets, tiles, ntiles, BM, shared_rows, split, row_token, slot_row);
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

hipError_t launch_route_permute_few(const float* partial, int S, const float* bias, int T, int E, int k, float scale,
                                    int32_t* ids, float* gates, float* logits, int32_t* ticket, int32_t* counts,
                                    int32_t* offsets, int32_t* row_token, int32_t* slot_row, int4* tiles,
                                    int32_t* ntiles, int BM, int shared_rows, const XcdSplit& split,
                                    hipStream_t stream) {
    route_permute_few_kernel<<<T, 256, 0, stream>>>(partial, S, bias, T, E, k, scale, ids, gates, logits, ticket,
                                                    counts, offsets, tiles, ntiles, BM, shared_rows, split, row_token,
                                                    slot_row);
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
