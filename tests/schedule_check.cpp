// CPU check of the work partition of the GEMM kernel (schedule.hpp),
// compiled with g++ by tests/test_schedule.py.
//
// For many (tiles, steps, grid) it replays the kernel's walk: every virtual
// workgroup v starts at range_begin(v) and computes segments tile by tile
// exactly as gemm_epi_kernel does.  It checks that
//   * virtual_wg is a permutation of the grid;
//   * every (tile, K step) iteration is computed exactly once;
//   * tile_segments(t) names exactly the workgroups that compute tile t, in
//     K order, and a tile is split iff it has more than one segment;
//   * partial_slot gives every segment of a split tile a distinct slot below
//     2 G (below G when G is a multiple of the tile count), and range_owner
//     agrees with the ranges;
//   * tile_coords is a bijection onto the tile grid;
//   * k_steps / k_offset cover K positions [0, K) exactly once.
#include <cstdint>
#include <cstdio>
#include <map>
#include <set>
#include <vector>

#include "schedule.hpp"

using namespace lin_epi;

static long g_fail = 0;
#define EXPECT(cond, ...)                          \
    do {                                           \
        if (!(cond)) {                             \
            if (g_fail < 20) {                     \
                std::printf("FAIL %s: ", #cond);   \
                std::printf(__VA_ARGS__);          \
                std::printf("\n");                 \
            }                                      \
            ++g_fail;                              \
        }                                          \
    } while (0)

static void check_partition(int tiles, int steps, int G)
{
    const int64_t T = (int64_t)tiles * steps;
    if (G > T) return;
    const int S = G % tiles == 0 ? G / tiles : 0;
    if (S > steps) return;  // the planner clamps S to the K steps
    const Partition p{steps, G, S, (int)(T / G), (int)(T % G)};
    std::vector<char> seen_v(G, 0);
    for (int w = 0; w < G; ++w) {
        const int v = virtual_wg(w, G);
        EXPECT(v >= 0 && v < G && !seen_v[v], "virtual_wg(%d, %d) = %d", w, G, v);
        if (v >= 0 && v < G) seen_v[v] = 1;
    }
    EXPECT(range_begin(p, 0) == 0 && range_begin(p, G) == T, "ranges cover [0, T) for G %d", G);
    std::vector<int> count(T, 0);
    std::map<int, std::vector<int>> segs;  // tile -> workgroups, in walk order
    std::map<int, std::vector<std::pair<int, int>>> seg_steps;
    std::set<int64_t> slots_used;
    for (int v = 0; v < G; ++v) {
        // the kernel's walk
        int it = range_begin(p, v);
        const int it_end = range_begin(p, v + 1);
        if (S == 0) EXPECT(it_end - it == p.q || it_end - it == p.q + 1, "range %d has %d iterations", v, it_end - it);
        if (S > 0) EXPECT(it_end - it >= steps / S && it_end - it <= steps / S + 1 && it / steps == (it_end - 1) / steps,
                          "split-K range %d: %d..%d", v, it, it_end);
        int t = it / steps;
        int s0 = it - t * steps;
        do {
            const int s1 = it_end - it < steps - s0 ? s0 + (it_end - it) : steps;
            it += s1 - s0;
            for (int s = s0; s < s1; ++s) ++count[(int64_t)t * steps + s];
            segs[t].push_back(v);
            seg_steps[t].push_back({s0, s1});
            EXPECT(s1 > s0, "empty segment of tile %d in range %d", t, v);
            for (int s = s0; s < s1; ++s) EXPECT(range_owner(p, t * steps + s) == v, "owner of (%d, %d)", t, s);
            ++t;
            s0 = 0;
        } while (it < it_end);
    }
    for (int64_t i = 0; i < T; ++i) EXPECT(count[i] == 1, "iteration %lld computed %d times", (long long)i, count[i]);
    for (auto &kv : segs) {
        const int t = kv.first;
        const auto &ws = kv.second;
        const TileSegs sg = tile_segments(p, t);
        if (S > 0) EXPECT((int)ws.size() == S, "split-K tile %d has %zu segments", t, ws.size());
        EXPECT(sg.first == ws.front() && sg.last == ws.back() && (int)ws.size() == sg.last - sg.first + 1,
               "segments of tile %d: %d..%d vs %zu", t, sg.first, sg.last, ws.size());
        for (size_t k = 0; k < ws.size(); ++k) {
            EXPECT(ws[k] == sg.first + (int)k, "segment %zu of tile %d", k, t);
            if (k > 0) EXPECT(seg_steps[t][k].first == seg_steps[t][k - 1].second, "K order of tile %d", t);
        }
        if (ws.size() > 1) {
            for (int u : ws) {
                const int64_t sl = partial_slot(p, u, t);
                EXPECT(sl >= 0 && sl < 2 * (int64_t)G, "slot %lld", (long long)sl);
                if (G % tiles == 0) EXPECT(sl < G, "split-K slot %lld beyond G", (long long)sl);
                EXPECT(slots_used.insert(sl).second, "slot %lld used twice (tile %d, workgroup %d)", (long long)sl, t, u);
            }
        }
    }
}

static void check_tiles(int tiles_m, int tiles_n)
{
    std::vector<char> hit((size_t)tiles_m * tiles_n, 0);
    for (int t = 0; t < tiles_m * tiles_n; ++t) {
        int tm, tn;
        tile_coords<8>(t, tiles_m, tiles_n, tm, tn);
        EXPECT(tm >= 0 && tm < tiles_m && tn >= 0 && tn < tiles_n, "tile %d -> (%d, %d)", t, tm, tn);
        if (tm >= 0 && tm < tiles_m && tn >= 0 && tn < tiles_n) {
            EXPECT(!hit[(size_t)tm * tiles_n + tn], "tile (%d, %d) twice", tm, tn);
            hit[(size_t)tm * tiles_n + tn] = 1;
        }
    }
}

static void check_k(int K)
{
    const int steps = k_steps(K), koff = k_offset(K);
    std::vector<int> cover(K > 0 ? K : 1, 0);
    for (int s = 0; s < steps; ++s)
        for (int k = koff + 32 * s; k < koff + 32 * s + 32; ++k) {
            if (k < 0 || k >= K) {
                EXPECT(k < 0 ? s == 0 : K == 0, "K %d: step %d position %d outside [0, K)", K, s, k);
                continue;
            }
            ++cover[k];
        }
    for (int k = 0; k < K; ++k) EXPECT(cover[k] == 1, "K %d: position %d covered %d times", K, k, cover[k]);
    EXPECT(koff <= 0 && koff > -32, "koff %d", koff);
}

int main()
{
    const int tile_counts[] = {1, 2, 3, 4, 7, 8, 32, 96, 128, 256, 376, 1000};
    const int step_counts[] = {1, 2, 3, 5, 16, 129, 256, 1024};
    for (int tiles : tile_counts)
        for (int steps : step_counts) {
            std::set<int> grids = {1, 2, 3, 7, 8, 9, 64, 255, 256, 257, 300, 512, 1000};
            for (int S = 1; S <= 16; ++S) grids.insert(tiles * S);
            for (int G : grids)
                if (G >= 1 && (int64_t)G <= (int64_t)tiles * steps && (int64_t)tiles * steps <= 2000000)
                    check_partition(tiles, steps, G);
        }
    const int shapes[][2] = {{1, 1}, {1, 7}, {4, 24}, {8, 47}, {9, 5}, {16, 64}, {3, 300}, {17, 17}};
    for (auto &sh : shapes) check_tiles(sh[0], sh[1]);
    for (int K = 0; K <= 300; K += 4) check_k(K);
    check_k(4100);
    check_k(32768);
    if (g_fail) {
        std::printf("%ld failures\n", g_fail);
        return 1;
    }
    std::printf("ok\n");
    return 0;
}
