// Host check of the chunk-walking matmul's workgroup schedule
// (tensor_gemm_collective_amd/csrc/coc_schedule.h) against brute-force
// definitions.  Built and run by tests/test_schedule_cpu.py; prints
// "cases N bad 0" on success.
#define COC_HD
#include "coc_schedule.h"

#include <cstdio>
#include <vector>

static int bad = 0;
#define CHECK(cond, ...)                                   \
    do {                                                   \
        if (!(cond)) {                                     \
            if (bad < 20) std::printf(__VA_ARGS__);        \
            ++bad;                                         \
        }                                                  \
    } while (0)

int main() {
    int cases = 0;
    unsigned r = 12345u;
    auto rnd = [&](unsigned n) { r = r * 1103515245u + 12345u; return (r >> 8) % n; };
    for (int iter = 0; iter < 4000; ++iter) {
        const int np = 1 + (int)rnd(9);
        const int per = 1 + (int)rnd(40);
        std::vector<int32_t> tiles(np), wait(np);
        int chunk = -1;
        for (int c = 0; c < np; ++c) {
            tiles[c] = (int32_t)rnd(iter % 3 == 0 ? 40 : 300);
            if (c > 0 && rnd(3) != 0) ++chunk;   // wait indices: -1, then non-decreasing chunks
            wait[c] = c == 0 ? -1 : (chunk < 0 ? 0 : chunk);
        }
        int singles_total = 0, early_ref = 0;
        std::vector<int> gatherer_seen;
        for (int x = 0; x < 8; ++x) {
            // the XCD's list, expanded: piece of each item, in order
            std::vector<int> list;
            for (int c = 0; c < np; ++c) {
                const int cnt = tiles[c] / 8 + (x < tiles[c] % 8 ? 1 : 0);
                for (int i = 0; i < cnt; ++i) list.push_back(c);
            }
            const int l = (int)list.size();
            CHECK(xcd_items(tiles.data(), 1, np, x) == l, "xcd_items x=%d\n", x);
            for (int j = 0; j < l; ++j) {
                int jj = -1;
                CHECK(piece_of_item(tiles.data(), 1, np, x, j, &jj) == list[j], "piece_of_item j=%d\n", j);
            }
            int jj = 0;
            CHECK(piece_of_item(tiles.data(), 1, np, x, l, &jj) == np, "piece_of_item past the end\n");

            // definition of the last-two-rounds split
            const int rounds = l > per ? (l + per - 1) / per : 1;
            const int base = l > per ? (rounds - 2) * per : 0;
            const int d = l > per ? l - base - per : -1;   // two-item workgroups of the last two rounds
            std::vector<int> seen(l, 0), seen_in(l, 0);
            for (int w = 0; w < per; ++w) {
                int last = -1, n = 0;
                for (int s = 0;; ++s) {
                    const int j = schedule_item(l, per, w, s);
                    if (j < 0) break;
                    CHECK(j < l && j > last, "schedule_item order l=%d per=%d w=%d s=%d j=%d\n", l, per, w, s, j);
                    if (j >= 0 && j < l) ++seen[j];
                    if (s == rounds - 2 && l > per) {   // first item of the last two rounds
                        if (w < d) CHECK(j == base + w, "two-tile first item\n");
                        else CHECK(j == base + 2 * d + (w - d), "one-tile item\n");
                    }
                    last = j;
                    ++n;
                }
                if (l <= per) CHECK(n == (w < l ? 1 : 0), "short list count\n");
                else CHECK(n == (w < d ? rounds : rounds - 1), "count l=%d per=%d w=%d n=%d\n", l, per, w, n);
                // in list order: item j at step j / per
                for (int s = 0;; ++s) {
                    const int j = inorder_item(l, per, w, s);
                    if (j < 0) break;
                    CHECK(j == w + s * per && j < l, "inorder_item\n");
                    ++seen_in[j];
                }
            }
            for (int j = 0; j < l; ++j) {
                CHECK(seen[j] == 1, "schedule_item covers item %d %d times (l=%d per=%d)\n", j, seen[j], l, per);
                CHECK(seen_in[j] == 1, "inorder_item covers item %d %d times\n", j, seen_in[j]);
            }
            // gatherers: one-tile workgroups of the last two rounds, numbered
            // before + (w - first) across the XCDs
            int first = -5;
            const int before = singles_before(tiles.data(), 1, np, per, x, &first);
            CHECK(before == singles_total, "singles_before x=%d\n", x);
            CHECK(first == (l > per ? d : -1), "first one-tile workgroup\n");
            if (l > per)
                for (int w = d; w < per; ++w) gatherer_seen.push_back(before + (w - d));
            singles_total += l > per ? per - d : 0;
            // early chunks by definition: pieces of the two-tile workgroups' first items
            if (l > per) {
                const int firsts = rounds >= 3 ? per : d;   // items 0 .. firsts-1
                for (int j = 0; j < firsts; ++j)
                    if (wait[list[j]] + 1 > early_ref) early_ref = wait[list[j]] + 1;
            }
        }
        int f = 0;
        CHECK(singles_before(tiles.data(), 1, np, per, 8, &f) == singles_total, "total one-tile workgroups\n");
        std::vector<int> hit(singles_total, 0);
        for (int g : gatherer_seen) {
            CHECK(g >= 0 && g < singles_total, "gatherer index range\n");
            if (g >= 0 && g < singles_total) ++hit[g];
        }
        for (int g = 0; g < singles_total; ++g) CHECK(hit[g] == 1, "gatherer %d numbered %d times\n", g, hit[g]);
        CHECK(early_chunks(tiles.data(), wait.data(), np, per) == early_ref, "early_chunks np=%d per=%d: %d vs %d\n",
              np, per, early_chunks(tiles.data(), wait.data(), np, per), early_ref);
        ++cases;
    }
    std::printf("cases %d bad %d\n", cases, bad);
    return bad != 0;
}
