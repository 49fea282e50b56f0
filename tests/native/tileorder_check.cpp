// Host-only check of the packed GEMM's work order (kq_tileorder.hpp):
//  1. every order is a cover: each tile once whole, or each of its halves once;
//  2. in a model of the dispatcher (workgroup i to XCD i % 8, each XCD's
//     workgroups in index order onto its ncu / 8 CUs, each to the CU that frees
//     first; a whole tile takes 2 time units, a half 1) the staggered order
//     finishes no later than the plain one;
//  3. a staggered order starts each XCD with both halves and whole tiles.
// Prints "ok" on success; the first failure is printed and exits 1.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "kq_tileorder.hpp"

using kq::g256::TileOrder;
using kq::g256::TileWork;

static void fail(const char *what, int nwg, int ncu, int i) {
    std::printf("FAIL %s nwg=%d ncu=%d i=%d\n", what, nwg, ncu, i);
    std::exit(1);
}

static int makespan(const TileOrder &o, int ncu) {
    const int groups = kq::g256::tile_order_groups(o);
    const int per_xcd = ncu / 8 > 0 ? ncu / 8 : 1;
    int worst = 0;
    for (int x = 0; x < 8; ++x) {
        std::vector<int> free_at(per_xcd, 0);
        for (int i = x; i < groups; i += 8) {
            int c = 0;
            for (int k = 1; k < per_xcd; ++k)
                if (free_at[k] < free_at[c]) c = k;
            free_at[c] += kq::g256::tile_work(i, o).half < 0 ? 2 : 1;
            if (free_at[c] > worst) worst = free_at[c];
        }
    }
    return worst;
}

int main() {
    const int ncus[] = {256, 304, 80, 64, 8, 1};
    int staggered_seen = 0;
    for (int ncu : ncus)
        for (int nwg = 1; nwg <= 4200; ++nwg) {
            const TileOrder o = kq::g256::make_tile_order(nwg, ncu);
            const int groups = kq::g256::tile_order_groups(o);
            std::vector<int> whole(nwg, 0), left(nwg, 0), right(nwg, 0);
            for (int i = 0; i < groups; ++i) {
                const TileWork w = kq::g256::tile_work(i, o);
                if (w.tile < 0 || w.tile >= nwg || w.half < -1 || w.half > 1) fail("range", nwg, ncu, i);
                (w.half < 0 ? whole : w.half == 0 ? left : right)[w.tile]++;
            }
            int split = 0;
            for (int t = 0; t < nwg; ++t) {
                const bool ok = (whole[t] == 1 && left[t] == 0 && right[t] == 0) ||
                                (whole[t] == 0 && left[t] == 1 && right[t] == 1);
                if (!ok) fail("cover", nwg, ncu, t);
                split += whole[t] == 0;
            }
            if (split != o.split) fail("split count", nwg, ncu, split);
            if (o.staggered) {
                ++staggered_seen;
                TileOrder plain = o;
                plain.staggered = 0;
                if (makespan(o, ncu) > makespan(plain, ncu)) fail("makespan", nwg, ncu, 0);
                for (int x = 0; x < 8; ++x) {
                    int halves = 0, wholes = 0;
                    for (int j = 0; j < ncu / 8; ++j)
                        (kq::g256::tile_work(8 * j + x, o).half < 0 ? wholes : halves)++;
                    if (halves == 0 || wholes == 0) fail("first round mix", nwg, ncu, x);
                }
            }
        }
    // the FLUX.1 projection 18432 x 3072 (72 x 12 tiles) on 256 CUs is staggered and
    // finishes in 3.5 tile times, as the plain order does
    const TileOrder f = kq::g256::make_tile_order(864, 256);
    TileOrder fp = f;
    fp.staggered = 0;
    if (!f.staggered || f.split != 96 || makespan(f, 256) != 7 || makespan(fp, 256) != 7) fail("flux", 864, 256, 0);
    if (staggered_seen < 100) fail("too few staggered cases", 0, 0, staggered_seen);
    std::printf("ok %d staggered orders checked\n", staggered_seen);
    return 0;
}
