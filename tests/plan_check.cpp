// Host-only check of the workspace layout: every region is large enough for what any launch plan may
// write into it (either grouped-GEMM kernel, any router split), and regions do not overlap.
// Built and run by tests/test_plan.py with g++ against the library's planner source.
#include <cstdio>
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
                        for (int Is : {0, I}) {
                            if (!moe::check_sizes(T, H, E, k, I, Is, true).ok()) continue;
                            ++n;
                            const moe::Layout L = moe::forward_layout(T, H, E, k, I, Is);
                            const size_t Tk = (size_t)T * k;
                            const size_t chunks = ((size_t)T + moe::kPermChunk - 1) / moe::kPermChunk;
                            const size_t tiles_need = (size_t)std::max(moe::max_tiles(T, E, k, moe::kSkinnyBM),
                                                                       moe::max_tiles(T, E, k, moe::kWideBM)) * 8;
                            struct R { size_t off, need; const char* name; };
                            std::vector<R> rs = {
                                {L.ids, Tk * 4, "ids"}, {L.gates, Tk * 4, "gates"}, {L.counts, (size_t)E * 4, "counts"},
                                {L.offsets, ((size_t)E + 1) * 4, "offsets"}, {L.row_token, Tk * 4, "row_token"},
                                {L.slot_row, Tk * 4, "slot_row"}, {L.chunk_base, chunks * E * 4, "chunk_base"},
                                {L.tiles, tiles_need, "tiles"}, {L.ntiles, 4, "ntiles"},
                                {L.partial, (size_t)moe::router_splits(T, H) * T * E * 4, "partial"},
                                {L.h_perm, Tk * I * 2, "h_perm"}, {L.y_perm, Tk * H * 4, "y_perm"}};
                            if (Is > 0) {
                                rs.push_back({L.h_sh, (size_t)T * Is * 2, "h_sh"});
                                rs.push_back({L.y_sh, (size_t)T * H * 4, "y_sh"});
                            }
                            for (size_t i = 0; i < rs.size(); ++i) {
                                const size_t end = i + 1 < rs.size() ? rs[i + 1].off : L.total;
                                CHECK(rs[i].off % 256 == 0, "%s offset %zu", rs[i].name, rs[i].off);
                                CHECK(end >= rs[i].off + rs[i].need, "T=%d H=%d E=%d k=%d I=%d Is=%d: %s has %zu < %zu",
                                      T, H, E, k, I, Is, rs[i].name, end - rs[i].off, rs[i].need);
                            }
                            const int S = moe::router_splits(T, H);
                            CHECK(S >= 1 && S <= H / 64, "splits %d for H=%d", S, H);
                        }
                }
    std::printf("%d layouts checked, %d failures\n", n, fails);
    return fails ? 1 : 0;
}
