// Work order of the packed-scale GEMM's launch: which output tile (or which
// half of one) each workgroup computes. Plain C++ (constexpr functions are
// callable from device code and from a host-only test build alike).
//
// Tiles are numbered in "run order": workgroups are dealt to the eight XCDs
// round robin (workgroup i to XCD i % 8), and each XCD's workgroups take a
// contiguous run of tile numbers, so the operand rows a run shares stay in that
// XCD's L2. A launch covers the tiles in whole rounds (one workgroup per CU);
// when the last round would leave at least half the CUs idle, its tiles are
// split into two 128-column halves instead, which evens the finish.
//
// Two orders:
//  - plain: the full tiles first, then the halves;
//  - staggered (when the numbers divide evenly over the XCDs): each XCD starts
//    its first round with half its CUs on halves and half on full tiles, keeps
//    the remaining halves for the end. The two groups of CUs then run half a
//    tile apart for the whole launch, so their output stores (the tile
//    epilogue, bound by HBM writes when every CU stores at once) alternate
//    instead of coinciding. The finish time in tile units is the same as the
//    plain order's.
#pragma once

namespace kq {
namespace g256 {

struct TileOrder {
    int nwg;           // tiles
    int split;         // tiles computed as two halves (0: none)
    int staggered;     // 1: staggered order (needs nwg, split, ncu all multiples of 8)
    int first_halves;  // staggered: halves per XCD at the start of its sequence (even)
};

struct TileWork {
    int tile;  // run-order tile number
    int half;  // -1: the whole tile; 0 or 1: its left or right 128 columns
};

// Number of workgroups the launch needs.
constexpr int tile_order_groups(const TileOrder &o) { return o.nwg + o.split; }

// The order for nwg tiles on ncu CUs.
constexpr TileOrder make_tile_order(int nwg, int ncu) {
    TileOrder o{nwg, 0, 0, 0};
    if (ncu <= 0 || nwg <= 0) return o;
    const int rem = nwg % ncu;
    if (rem == 0 || 2 * rem > ncu) return o;  // whole rounds, or a last round at least half full
    o.split = rem;
    if (nwg > rem && nwg % 8 == 0 && rem % 8 == 0 && ncu % 8 == 0) {  // at least one whole round
        const int halves = 2 * (rem / 8), cus = ncu / 8;
        int h1 = halves < cus / 2 ? halves : cus / 2;
        h1 &= ~1;
        if (h1 > 0) {
            o.staggered = 1;
            o.first_halves = h1;
        }
    }
    return o;
}

// Workgroup i's tile (plain order: tile numbers remapped to XCD runs here).
constexpr TileWork tile_work(int i, const TileOrder &o) {
    if (o.staggered) {
        const int x = i % 8, j = i / 8;
        const int per = o.nwg / 8, rx = o.split / 8, full = per - rx, h1 = o.first_halves;
        TileWork w{0, -1};
        if (j < h1) {
            w.tile = full + j / 2;
            w.half = j % 2;
        } else if (j < h1 + full) {
            w.tile = j - h1;
        } else {
            const int k = j - full;
            w.tile = full + k / 2;
            w.half = k % 2;
        }
        w.tile += x * per;
        return w;
    }
    const int nfull = o.nwg - o.split;
    int p = i, half = -1;
    if (i >= nfull) {
        p = nfull + (i - nfull) / 2;
        half = (i - nfull) % 2;
    }
    const int q = o.nwg / 8, rm = o.nwg % 8, x = p % 8, loc = p / 8;
    const int tile = x < rm ? x * (q + 1) + loc : rm * (q + 1) + (x - rm) * q + loc;
    return TileWork{tile, half};
}

}  // namespace g256
}  // namespace kq
