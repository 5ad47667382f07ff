// Host-only check of the workspace layout: every region is large enough for what any launch plan may
// write into it (either grouped-GEMM kernel, any router split), and regions do not overlap.
// Built and run by tests/test_plan.py with g++ against the library's planner source.
#include <cstdio>
#include <algorithm>
#include <cstdint>
#include <cstdlib>
#include <vector>

#include "plan.h"

static int fails = 0;
#define CHECK(c, ...)                                             \
    do {                                                          \
        if (!(c)) {                                               \
            std::printf("FAIL %s: ", #c);                        \
            std::printf(__VA_ARGS__);                             \
            std::printf("\n");                                    \
            ++fails;                                              \
        }                                                         \
    } while (0)

int main() {
    const int Ts[] = {1, 7, 16, 64, 129, 384, 1000, 4096, 8192, 32768};
    const int Hs[] = {64, 192, 2048, 6144};
    const int Es[] = {1, 8, 16, 24, 64, 256};
    const int ks[] = {1, 4, 8, 32};
    const int Is_[] = {64, 1536, 2048};
    int n = 0;
    for (int T : Ts)
        for (int H : Hs)
            for (int E : Es)
                for (int k : ks) {
                    if (k > E) continue;
                    for (int I : Is_)
                        for (int Is : {0, I, 2 * I}) {
                            if (!moe::check_sizes(T, H, E, k, I, Is, true).ok()) continue;
                            ++n;
                            const moe::Layout L = moe::forward_layout(T, H, E, k, I, Is, true);
                            const moe::Layout L0 = moe::forward_layout(T, H, E, k, I, Is);
                            CHECK(L0.y_perm == L.y_perm && L0.x_norm == size_t(-1) && L0.total <= L.x_norm,
                                  "the norm region must only extend the plain layout");
                            const size_t Tk = (size_t)T * k;
                            const size_t chunks = ((size_t)T + moe::kPermChunk - 1) / moe::kPermChunk;
                            // the shared expert with the routed width is one more group of the routed GEMMs:
                            // T more rows in h_perm / y_perm and its tiles after the routed ones
                            const bool fold = moe::shared_fold(T, E, k, I, Is);
                            CHECK(fold == (Is == I && (int64_t)T * k <= (int64_t)moe::kSkinnyBM * E),
                                  "fold T=%d E=%d k=%d I=%d Is=%d", T, E, k, I, Is);
                            const size_t rows = Tk + (fold ? (size_t)T : 0);
                            size_t tiles_need = 0;
                            for (int BM : {moe::kSkinnyBM, moe::kWideBM, moe::kTallBM})
                                tiles_need = std::max(tiles_need, (size_t)(moe::max_tiles(T, E, k, BM) +
                                                                           (fold ? moe::shared_tiles(T, BM) : 0)) *
                                                                  moe::kTileEntryBytes);
                            struct R { size_t off, need; const char* name; };
                            std::vector<R> rs = {
                                {L.ids, Tk * 4, "ids"}, {L.gates, Tk * 4, "gates"}, {L.counts, (size_t)E * 4, "counts"},
                                {L.offsets, ((size_t)E + 1) * 4, "offsets"}, {L.row_token, Tk * 4, "row_token"},
                                {L.slot_row, Tk * 4, "slot_row"}, {L.chunk_base, chunks * E * 4, "chunk_base"},
                                {L.tiles, tiles_need, "tiles"}, {L.ntiles, 4, "ntiles"},
                                {L.partial, (size_t)moe::router_splits(T, H, E) * T * E * 4, "partial"},
                                {L.h_perm, (Tk + (Is == I ? (size_t)T : 0)) * I * 2, "h_perm"},
                                {L.y_perm, rows * H * (moe::slot_rows_bf16(T, E, k, I, Is) ? 2 : 4), "y_perm"}};
                            // shared rows outside the decode fold: y_shared fp32 [T, H]; h in the rows after the
                            // routed ones when Is == I, else a region of its own
                            CHECK((L.y_sh == size_t(-1)) == (fold || Is == 0) &&
                                      (L.h_sh == size_t(-1)) == (fold || Is == 0 || Is == I),
                                  "shared buffers (T=%d E=%d k=%d I=%d Is=%d)", T, E, k, I, Is);
                            if (Is > 0 && !fold) {
                                if (Is != I) rs.push_back({L.h_sh, (size_t)T * Is * 2, "h_sh"});
                                rs.push_back({L.y_sh, (size_t)T * H * 4, "y_sh"});
                            }
                            if (L.sh_partial != size_t(-1))
                                rs.push_back({L.sh_partial, moe::dense_partial_bytes(T, H, Is), "sh_partial"});
                            CHECK((L.ks_flag != size_t(-1)) == moe::ksplit_possible(T, H, E, k, I, Is) &&
                                      (L.ks_part != size_t(-1)) == (L.ks_flag != size_t(-1)),
                                  "K-split regions (T=%d E=%d k=%d I=%d Is=%d)", T, E, k, I, Is);
                            CHECK((L.ks_part_down != size_t(-1)) == (L.ks_flag != size_t(-1)), "K-split down rows");
                            // bf16 per-slot rows never meet a K split or folded shared rows, and need 8 slots
                            CHECK(!moe::slot_rows_bf16(T, E, k, I, Is) ||
                                      (!fold && k >= 8 && !moe::ksplit_possible(T, H, E, k, I, Is)),
                                  "bf16 per-slot rows (T=%d E=%d k=%d)", T, E, k);
                            if (L.ks_flag != size_t(-1)) {
                                rs.push_back({L.ks_flag, 16, "ks_flag"});
                                rs.push_back({L.ks_part, 2 * rows * I * 2 * 4, "ks_part"});
                                rs.push_back({L.ks_part_down, (size_t)(moe::down_split_max(T) - 1) * rows * H * 4,
                                              "ks_part_down"});
                            }
                            rs.push_back({L.x_norm, (size_t)T * H * 2, "x_norm"});
                            for (size_t i = 0; i < rs.size(); ++i) {
                                const size_t end = i + 1 < rs.size() ? rs[i + 1].off : L.total;
                                CHECK(rs[i].off % 256 == 0, "%s offset %zu", rs[i].name, rs[i].off);
                                CHECK(end >= rs[i].off + rs[i].need, "T=%d H=%d E=%d k=%d I=%d Is=%d: %s has %zu < %zu",
                                      T, H, E, k, I, Is, rs[i].name, end - rs[i].off, rs[i].need);
                            }
                            const int S = moe::router_splits(T, H, E);
                            CHECK(S >= 1 && S <= moe::kRouterMaxSplits && S <= (T <= moe::kRouterSmallT ? H / 32 : H / 64),
                                  "splits %d for T=%d H=%d", S, T, H);
                        }
                }
    // Workgroup order of the LDS-tiled grouped GEMM: with the grid padded to a multiple of kXcds, every
    // (tile, column tile) pair of the live tile list is taken by exactly one workgroup, each XCD's
    // workgroups cover a contiguous range of the order, and an expert's pairs are contiguous in it.
    uint64_t rng = 0x9E3779B97F4A7C15ull;
    auto next = [&]() {
        rng ^= rng << 13;
        rng ^= rng >> 7;
        rng ^= rng << 17;
        return rng;
    };
    int orders = 0;
    for (int trial = 0; trial < 300; ++trial) {
        const int E = 1 + (int)(next() % 64);
        const int k = 1 + (int)(next() % std::min(E, 8));
        const int T = (int)(next() % 2000);
        const int ntn = 1 + (int)(next() % 40);
        const int BM = trial % 2 ? moe::kWideBM : moe::kTallBM;
        // every other trial with a folded shared expert: group E, all T tokens, its tiles last
        const bool shared = trial % 4 < 2;
        std::vector<int> counts(E + 1, 0);
        const bool skew = trial % 3 == 0;
        for (int t = 0; t < T * k; ++t) counts[skew ? (int)(next() % 4) % E : (int)(next() % E)]++;
        counts[E] = shared ? T : 0;
        // tiles in chunks (plain: up to kMaxChunkTiles per chunk; every third trial the dealt sizes), each
        // entry packed as the device writes it: {tile_word, first row}
        std::vector<std::pair<int, int>> tiles; // {expert, first row}
        std::vector<int> words;
        std::vector<int> height(E + 1);
        for (int e = 0; e <= E; ++e) {
            height[e] = moe::tile_height(counts[e], BM);
            const int nt = counts[e] > 0 ? (counts[e] + height[e] - 1) / height[e] : 0;
            const int nc = trial % 3 == 1 ? moe::dealt_chunks(nt) : moe::plain_chunks(nt);
            for (int c = 0; c < nc; ++c) {
                const int f = moe::chunk_first(c, nc, nt), cm = moe::chunk_first(c + 1, nc, nt) - f;
                CHECK(cm >= 1 && cm <= moe::kMaxChunkTiles, "chunk of %d tiles", cm);
                for (int ci = 0; ci < cm; ++ci) {
                    tiles.push_back({e, (f + ci) * height[e]});
                    const int w = moe::tile_word(e, height[e], ci, cm);
                    CHECK(moe::tile_group(w) == e && moe::tile_ht(w) == height[e] && moe::tile_ci(w) == ci &&
                              moe::tile_cm(w) == cm, "tile word e=%d ht=%d ci=%d cm=%d", e, height[e], ci, cm);
                    words.push_back(w);
                }
            }
        }
        const int64_t live = (int64_t)tiles.size() * ntn;
        int64_t grid = (moe::max_tiles(T, E, k, BM) + (shared ? moe::shared_tiles(T, BM) : 0)) * ntn;
        CHECK(grid >= live, "grid %lld < live %lld", (long long)grid, (long long)live);
        grid = (grid + moe::kXcds - 1) / moe::kXcds * moe::kXcds;
        std::vector<int> seen(live, 0);
        std::vector<int64_t> lo(moe::kXcds, INT64_MAX), hi(moe::kXcds, -1), cnt(moe::kXcds, 0);
        for (int64_t b = 0; b < grid; ++b) {
            const int64_t L = moe::xcd_block_order(b, live);
            if (L < 0) continue;
            const int x = (int)(b % moe::kXcds);
            lo[x] = std::min(lo[x], L);
            hi[x] = std::max(hi[x], L);
            ++cnt[x];
            const auto entry = tiles[L / ntn];
            const int w = words[L / ntn];
            int nt = -1;
            const int64_t mt = moe::chunk_major_tile(L, ntn, moe::tile_ci(w), moe::tile_cm(w), nt);
            CHECK(mt >= 0 && mt < (int64_t)tiles.size() && tiles[mt].first == entry.first,
                  "block %lld: tile %lld outside expert %d", (long long)b, (long long)mt, entry.first);
            // the device derives the block's first row from the entry it read and the tile distance
            if (mt >= 0 && mt < (int64_t)tiles.size())
                CHECK(entry.second + (mt - L / ntn) * moe::tile_ht(w) == tiles[mt].second, "first row of tile %lld",
                      (long long)mt);
            CHECK(nt >= 0 && nt < ntn, "block %lld: column tile %d of %d", (long long)b, nt, ntn);
            if (mt >= 0 && mt < (int64_t)tiles.size() && nt >= 0 && nt < ntn) seen[mt * ntn + nt]++;
        }
        for (int64_t i = 0; i < live; ++i) CHECK(seen[i] == 1, "pair %lld taken %d times", (long long)i, seen[i]);
        for (int x = 0; x < moe::kXcds; ++x)
            CHECK(cnt[x] == 0 || hi[x] - lo[x] + 1 == cnt[x], "XCD %d range not contiguous", x);
        ++orders;
    }
    std::printf("%d block orders checked\n", orders);

    // the dealt order: chunk c goes to slot deal_slot(c) of XCD deal_xcd(c); every (XCD, slot) is taken once,
    // in dealing order within an XCD, and the XCDs take turns in snake order
    {
        std::vector<int> owner(moe::kXcds * moe::kDealtSlots, -1);
        std::vector<int> last(moe::kXcds, -1);
        for (int c = 0; c < moe::kMaxDealtChunks; ++c) {
            const int x = moe::deal_xcd(c), sl = moe::deal_slot(c);
            CHECK(x >= 0 && x < moe::kXcds && sl >= 0 && sl < moe::kDealtSlots, "chunk %d -> (%d, %d)", c, x, sl);
            if (x < 0 || x >= moe::kXcds || sl < 0 || sl >= moe::kDealtSlots) continue;
            CHECK(owner[x * moe::kDealtSlots + sl] == -1, "slot (%d, %d) taken twice", x, sl);
            owner[x * moe::kDealtSlots + sl] = c;
            CHECK(sl == last[x] + 1, "XCD %d slots out of order at chunk %d", x, c);
            last[x] = sl;
        }
        CHECK(moe::deal_xcd(7) == 7 && moe::deal_xcd(8) == 7 && moe::deal_xcd(15) == 0 && moe::deal_xcd(16) == 0,
              "snake dealing");
        // chunks per group: at least one per 128 tiles, at most 8 for groups up to 1024 tiles
        for (int nt = 1; nt <= 5000; ++nt) {
            const int nc = moe::dealt_chunks(nt), pc = moe::plain_chunks(nt);
            CHECK(nc >= 1 && (nt > 1024 || nc <= 8) && (nt + nc - 1) / nc <= moe::kMaxChunkTiles &&
                      (nt < 32 || nc >= 8 || nt > 1024) && pc == (nt + 127) / 128,
                  "chunks of %d tiles: dealt %d, plain %d", nt, nc, pc);
        }
    }

    // workspace queries: the largest layout over every T' <= T, so a workspace sized for the largest batch
    // serves every smaller one (brute force over T' for small T, sampled T up to past the split ranges)
    {
        struct Shape { int H, E, k, I, Is; };
        const Shape shapes[] = {{6144, 256, 8, 2048, 2048}, {2048, 64, 4, 1536, 1536}, {256, 16, 4, 128, 128},
                                {192, 8, 8, 64, 0}, {256, 32, 1, 128, 192}, {64, 1, 1, 64, 64},
                                {6144, 256, 8, 2048, 0}, {128, 4, 2, 128, 128}};
        for (const Shape& q : shapes) {
            for (int norm = 0; norm < 2; ++norm) {
                size_t run = 0, prev = 0;
                for (int T = 0; T <= 40000; ++T) {
                    run = std::max(run, moe::forward_layout(T, q.H, q.E, q.k, q.I, q.Is, norm).total);
                    if (T > 1500 && T % 97 != 0 && T != 32768 && T != 32769) continue;
                    const size_t b = moe::forward_workspace_bound(T, q.H, q.E, q.k, q.I, q.Is, norm);
                    CHECK(b == run && b >= prev, "forward bound T=%d H=%d E=%d k=%d I=%d Is=%d norm=%d: %zu vs %zu",
                          T, q.H, q.E, q.k, q.I, q.Is, norm, b, run);
                    prev = b;
                }
            }
            size_t run = 0;
            for (int T = 0; T <= 20000; ++T) {
                run = std::max(run, moe::dense_workspace_bytes(T, q.H, q.I));
                if (T > 1500 && T % 97 != 0) continue;
                CHECK(moe::dense_workspace_bound(T, q.H, q.I) == run, "dense bound T=%d H=%d I=%d", T, q.H, q.I);
            }
        }
    }

    // K split of decode-sized gate/up launches: split when two half-length rounds beat one (5 % margin)
    CHECK(moe::decode_ksplit(1312, 256) == 2 && moe::decode_ksplit(1536, 256) == 1 &&
              moe::decode_ksplit(272, 256) == 2 && moe::decode_ksplit(144, 256) == 1 &&
              moe::decode_ksplit(17, 256) == 1 && moe::decode_ksplit(0, 256) == 1 &&
              moe::decode_ksplit(100, 0) == 1,
          "decode_ksplit");
    // the down GEMM's rule: among the allowed splits the fewest rounds per unit of work, two ranges already at
    // a tie with one, each range beyond two 5 % dearer
    for (int64_t b = 0; b < 5000; b += 7)
        for (int cus : {80, 256, 304}) {
            const int64_t r1 = (b + cus - 1) / cus;
            const int s = moe::decode_ksplit_down(b, cus, (1 << 2) | (1 << 3) | (1 << 4));
            CHECK(s >= 1 && s <= moe::kMaxDownSplits, "decode_ksplit_down range");
            CHECK(r1 >= 2 || s == 1, "decode_ksplit_down splits one round b=%lld", (long long)b);
            if (s > 1) { // no worse than one range
                const int64_t rs = (s * b + cus - 1) / cus;
                CHECK(rs * (18 + s) <= r1 * 20 * s, "decode_ksplit_down beats one range b=%lld", (long long)b);
            }
            CHECK(moe::decode_ksplit_down(b, cus, 0) == 1, "decode_ksplit_down without splits");
            CHECK(moe::decode_ksplit_down(b, cus, 1 << 2) == (r1 >= 2 && (2 * b + cus - 1) / cus <= 2 * r1 ? 2 : 1),
                  "decode_ksplit_down two-way b=%lld", (long long)b);
        }
    // GLM-4.7-Flash decode's down GEMM (296 blocks): 3 ranges when 2 and 3 are allowed (the streamed kernel's
    // whole ring periods of 24 K steps), 4 with 4 allowed; GLM-5 decode's (1968 blocks) in two
    CHECK(moe::decode_ksplit_down(296, 256, (1 << 2) | (1 << 3)) == 3 &&
              moe::decode_ksplit_down(296, 256, (1 << 2) | (1 << 3) | (1 << 4)) == 4 &&
              moe::decode_ksplit_down(1968, 256, (1 << 2) | (1 << 3) | (1 << 4)) == 2,
          "decode_ksplit_down GLM shapes");
    CHECK(moe::down_split_max(16) == moe::kMaxDownSplits && moe::down_split_max(17) == 2, "down_split_max");
    // streamed decode GEMMs: GLM-4.7-Flash decode (42 groups: 504 gate/up, 336 down blocks) yes, GLM-5 decode
    // (102 groups: 1632 gate/up, 816 down blocks, K split in two) no
    CHECK(moe::decode_streamed(504, 256) && moe::decode_streamed(336, 256) && !moe::decode_streamed(1632, 256) &&
              !moe::decode_streamed(816, 256) && !moe::decode_streamed(0, 256) && !moe::decode_streamed(10, 0),
          "decode_streamed");
    for (int64_t b = 1; b < 5000; b += 7)
        for (int cus : {80, 256, 304}) {
            const int64_t r1 = (b + cus - 1) / cus, r2 = (2 * b + cus - 1) / cus;
            CHECK(moe::decode_ksplit(b, cus) == (r1 >= 2 && 0.525 * (double)r2 < (double)r1 ? 2 : 1),
                  "split b=%lld cus=%d", (long long)b, cus);
        }
    // expected experts reached at decode: GLM-5 at 16 tokens (top-8 of 256) about 101, GLM-4.7-Flash (top-4 of
    // 64) about 41; the gate/up GEMM splits K at the first and not at the second on 256 CUs
    CHECK(moe::expected_active(16, 256, 8) == 101 && moe::expected_active(16, 64, 4) == 41 &&
              moe::expected_active(1, 256, 8) == 8 && moe::expected_active(100000, 64, 4) == 64 &&
              moe::expected_active(0, 64, 4) == 0,
          "expected_active");
    CHECK(moe::decode_ksplit((int64_t)(101 + 1) * 16, 256) == 2 && moe::decode_ksplit((int64_t)(41 + 1) * 12, 256) == 1,
          "decode gate/up split at GLM-5 / GLM-4.7-Flash");
    // four ranges: only where two already pay, half-length blocks take at least 8 rounds and quarter-length
    // ones round strictly better (GLM-5 decode, 81 groups x 16 column tiles: 11 rounds of halves, 21 of quarters)
    CHECK(moe::decode_ksplit_gate_up(1296, 256, true) == 4 && moe::decode_ksplit_gate_up(1296, 256, false) == 2 &&
              moe::decode_ksplit_gate_up(1152, 256, true) == 2 && moe::decode_ksplit_gate_up(444, 256, true) == 1 &&
              moe::decode_ksplit_gate_up(600, 256, true) == 2 && moe::decode_ksplit_gate_up(0, 256, true) == 1,
          "decode_ksplit_gate_up");
    for (int64_t b = 1; b < 5000; b += 7)
        for (int cus : {80, 256, 304}) {
            const int s2 = moe::decode_ksplit(b, cus), s4 = moe::decode_ksplit_gate_up(b, cus, true);
            const int64_t r2 = (2 * b + cus - 1) / cus, r4 = (4 * b + cus - 1) / cus;
            CHECK(s4 == (s2 == 2 && r2 >= 8 && r4 < 2 * r2 ? 4 : s2) && moe::decode_ksplit_gate_up(b, cus, false) == s2,
                  "gate/up split b=%lld cus=%d", (long long)b, cus);
        }
    // block claims of the persistent kernel: any interleaving of front (home) and back (other XCDs) claims
    // hands every block of the range out exactly once, and later claims get none
    {
        uint64_t rng = 12345;
        auto next = [&]() { rng = rng * 6364136223846793005ull + 1442695040888963407ull; return rng >> 33; };
        for (int trial = 0; trial < 2000; ++trial) {
            const int lo = (int)(next() % 1000), n = (int)(next() % 300);
            std::vector<int> seen(n, 0);
            uint64_t ctr = 0; // the claims reach the counter in some order; each sees the sum before it
            int got = 0;
            const int claims = n + (int)(next() % 20);
            const int back_pct = (int)(next() % 101);
            for (int c = 0; c < claims; ++c) {
                const bool home = (int)(next() % 100) >= back_pct;
                const uint64_t old = ctr;
                ctr += home ? moe::kClaimFront : moe::kClaimBack;
                const int64_t b = moe::claim_block(lo, lo + n, old, home);
                if (c < n) {
                    CHECK(b >= lo && b < lo + n, "claim %d of %d got %lld", c, n, (long long)b);
                    if (b >= lo && b < lo + n) seen[b - lo]++, got++;
                } else {
                    CHECK(b == -1, "claim %d past %d blocks got %lld", c, n, (long long)b);
                }
            }
            for (int i = 0; i < n; ++i) CHECK(seen[i] == 1, "block %d of %d claimed %d times", i, n, seen[i]);
            CHECK(got == n, "%d of %d blocks claimed", got, n);
        }
    }
    // tile heights: at most BM, never more tiles than ceil(n / BM), no empty last tile; for the LDS-tiled
    // kernel a multiple of 16 rows (128) or 32 rows (256), the last tile shorter by less than that per tile
    for (int BM : {moe::kSkinnyBM, moe::kWideBM, moe::kTallBM})
        for (int n = 1; n <= 40000; n += (n < 3000 ? 1 : 97)) {
            const int ht = moe::tile_height(n, BM);
            const int nt = (n + ht - 1) / ht;
            CHECK(ht > 0 && ht <= BM && nt <= (n + BM - 1) / BM && (nt - 1) * ht < n, "n=%d BM=%d ht=%d", n, BM, ht);
            if (BM != moe::kSkinnyBM) {
                const int q = BM == moe::kTallBM ? 32 : 16;
                CHECK(ht % q == 0, "n=%d BM=%d height %d", n, BM, ht);
                const int last = n - (nt - 1) * ht;
                CHECK(nt == 1 || ht - last < q * nt, "n=%d BM=%d uneven tiles (height %d, last %d)", n, BM, ht, last);
            } else {
                CHECK(ht == BM, "n=%d BM=%d height %d", n, BM, ht);
            }
        }

    // split dense GEMMs on the weight-streaming kernel: every K range is non-empty and the partial region
    // holds both GEMMs' partials; a forward layout with a shared expert holds them too
    int dense = 0;
    for (int T : {1, 7, 16, 64, 129, 384, 1000, 4096})
        for (int H : {64, 256, 2048, 6144})
            for (int Id : {64, 384, 1536, 2048, 10240, 12288}) {
                ++dense;
                const int s1 = moe::dense_splits(true, T, Id, H), s2 = moe::dense_splits(false, T, H, Id);
                CHECK(s1 >= 1 && s1 <= moe::kMaxDenseSplits && (s1 == 1 || H / 64 >= s1),
                      "gate/up splits %d (T=%d H=%d I=%d)", s1, T, H, Id);
                CHECK(s2 >= 1 && s2 <= moe::kMaxDenseSplits && (s2 == 1 || Id / 64 >= s2),
                      "down splits %d (T=%d H=%d I=%d)", s2, T, H, Id);
                const size_t need = std::max(s1 > 1 ? (size_t)s1 * T * 2 * Id * 4 : 0,
                                             s2 > 1 ? (size_t)s2 * T * H * 4 : 0);
                CHECK(moe::dense_partial_bytes(T, H, Id) >= need, "partials T=%d H=%d I=%d", T, H, Id);
                // the LDS-copy kernel's splits at few rows, on any CU count: 4 K steps per range at least, and
                // partials within the same region
                for (int cus : {1, 80, 256, 304, 1024}) {
                    const int d1 = moe::dma_dense_splits(true, T, Id, H, cus), d2 = moe::dma_dense_splits(false, T, H, Id, cus);
                    CHECK(d1 >= 1 && d1 <= moe::kMaxDenseSplits && (d1 == 1 || (H / 64) / d1 >= 4) &&
                              (T <= moe::kDmaSplitMaxT || d1 == 1),
                          "dma gate/up splits %d (T=%d H=%d I=%d cus=%d)", d1, T, H, Id, cus);
                    CHECK(d2 >= 1 && d2 <= moe::kMaxDenseSplits && (d2 == 1 || (Id / 64) / d2 >= 4) &&
                              (T <= moe::kDmaSplitMaxT || d2 == 1),
                          "dma down splits %d (T=%d H=%d I=%d cus=%d)", d2, T, H, Id, cus);
                    const size_t nd = std::max(d1 > 1 ? (size_t)d1 * T * 2 * Id * 4 : 0, d2 > 1 ? (size_t)d2 * T * H * 4 : 0);
                    CHECK(moe::dense_partial_bytes(T, H, Id) >= nd, "dma partials T=%d H=%d I=%d", T, H, Id);
                    // the streamed form: ranges of a whole number of ring periods (4 K steps), within the same
                    // partial region; 0 exactly when K / 64 is not a multiple of 4
                    const int e1 = moe::dma_stream_splits(true, T, Id, H, cus), e2 = moe::dma_stream_splits(false, T, H, Id, cus);
                    CHECK((e1 == 0) == ((H / 64) % 4 != 0) && (e2 == 0) == ((Id / 64) % 4 != 0),
                          "stream splits defined (T=%d H=%d I=%d cus=%d)", T, H, Id, cus);
                    CHECK(e1 <= moe::kMaxDenseSplits && (e1 <= 1 || ((H / 64) / 4) % e1 == 0) &&
                              (T <= moe::kDmaSplitMaxT || e1 <= 1),
                          "stream gate/up splits %d (T=%d H=%d I=%d cus=%d)", e1, T, H, Id, cus);
                    CHECK(e2 <= moe::kMaxDenseSplits && (e2 <= 1 || ((Id / 64) / 4) % e2 == 0) &&
                              (T <= moe::kDmaSplitMaxT || e2 <= 1),
                          "stream down splits %d (T=%d H=%d I=%d cus=%d)", e2, T, H, Id, cus);
                    const size_t ne = std::max(e1 > 1 ? (size_t)e1 * T * 2 * Id * 4 : 0, e2 > 1 ? (size_t)e2 * T * H * 4 : 0);
                    CHECK(moe::dense_partial_bytes(T, H, Id) >= ne, "stream partials T=%d H=%d I=%d", T, H, Id);
                }
                // GLM-5 dense MLP at 16 tokens on 256 CUs: 96 gate/up blocks in ranges that fill whole rounds
                CHECK(moe::dma_dense_splits(true, 16, 12288, 6144, 256) >= 5 &&
                          moe::dma_dense_splits(false, 16, 6144, 12288, 256) >= 8, "GLM-5 dense splits");
                // streamed: one round filling three quarters of the CUs: 96 gate/up blocks x 2 ranges of 48 steps,
                // 24 down blocks x 8 ranges of 24 steps (192 blocks each)
                CHECK(moe::dma_stream_splits(true, 16, 12288, 6144, 256) == 2 &&
                          moe::dma_stream_splits(false, 16, 6144, 12288, 256) == 8, "GLM-5 dense stream splits");
                CHECK(moe::dense_workspace_bytes(T, H, Id) >= (size_t)T * Id * 2 + need, "dense workspace");
                const moe::Layout L = moe::forward_layout(T, H, 8, 2, Id == 64 ? 128 : 64, Id);
                CHECK(need == 0 || (L.sh_partial != size_t(-1) && L.x_norm == size_t(-1) &&
                                    L.total >= L.sh_partial + need),
                      "shared partials T=%d H=%d Is=%d", T, H, Id);
            }
    std::printf("%d dense splits checked\n", dense);

    // the DMA kernel's 32-bit byte offsets: a matrix fits while rows * K * 2 < 2^32, exactly at the edge;
    // the grouped GEMMs default to the DMA kernel, dense ones of up to 16 rows to the weight-streaming
    // kernel; the fallback picks by rows per expert
    CHECK(moe::dma_fits(1, 64) && moe::dma_fits(8192, 6144) && moe::dma_fits(589824, 2048), "dma_fits small");
    CHECK(moe::dma_fits((int64_t(1) << 31) / 6144, 6144) && !moe::dma_fits((int64_t(1) << 31) / 4096 + 1, 4096) &&
              moe::dma_fits((int64_t(1) << 31) / 4096, 4096 - 1) && !moe::dma_fits(int64_t(1) << 20, 4096),
          "dma_fits edge");
    for (int T : {1, 16, 17, 64, 1000, 8192})
        for (int E : {1, 16, 64, 256})
            for (int k : {1, 4, 8}) {
                if (k > E) continue;
                const moe::GemmPath p = moe::gemm_path(T, E, k), f = moe::fallback_path(T, E, k);
                const bool skinny = (int64_t)T * k <= (int64_t)moe::kSkinnyBM * E;
                CHECK(p == moe::GemmPath::Dma, "path T=%d E=%d k=%d", T, E, k);
                CHECK(moe::dense_path(T) == moe::GemmPath::Dma, "dense path T=%d", T);
                CHECK(skinny ? f == moe::GemmPath::Skinny : (f == moe::GemmPath::Wide || f == moe::GemmPath::Tall),
                      "fallback T=%d E=%d k=%d", T, E, k);
                CHECK(moe::path_bm(moe::GemmPath::Dma) == moe::kTallBM, "dma tile height");
            }
    std::printf("%d layouts checked, %d failures\n", n, fails);
    return fails ? 1 : 0;
}
