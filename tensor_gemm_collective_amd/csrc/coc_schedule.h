// Workgroup schedule of the chunk-walking matmul: which tiles each
// workgroup runs, in which order.  Shared by the kernels (device) and the
// host code that sets counter targets from the same schedule; plain C++ so a
// CPU test can check it exhaustively.  The includer defines COC_HD (the
// function qualifiers: __host__ __device__ for HIP, empty for a host build).
#ifndef COC_SCHEDULE_H
#define COC_SCHEDULE_H

#include <stdint.h>

#ifndef COC_HD
#error "define COC_HD before including coc_schedule.h"
#endif

// The launch has 8 * per_xcd workgroups; workgroup b runs on the XCD shared
// by every b' = b mod 8 and is workgroup w = b / 8 of that XCD.  Each XCD
// walks its own list of l tiles: piece by piece, each piece's tiles split
// into 8 runs, one per XCD.

// Items of XCD x's list (the pieces' tiles split over the 8 XCDs).
// (A piece has tiles_m[c] * tiles_n tiles.)
COC_HD inline int xcd_items(const int32_t* tiles_m, int tiles_n, int npieces, int x) {
    int l = 0;
    for (int c = 0; c < npieces; ++c) {
        const int t = tiles_m[c] * tiles_n;
        l += t / 8 + (x < t % 8 ? 1 : 0);
    }
    return l;
}

// The s-th item of workgroup w among per_xcd on a list of l items, or -1.
// Whole rounds first (w, w + per_xcd, ...); the last two rounds, with
// l' items, have d = l' - per_xcd workgroups doing two items and the rest
// one: the two-item workgroups take the first d items and then the next d,
// the one-item workgroups the last ones.  List order is chunk order, so the
// workgroups that must also finish a second tile start on the chunks that
// are ready first, and those that start last have a whole tile of slack.
COC_HD inline int schedule_item(int l, int per_xcd, int w, int s) {
    if (l <= per_xcd) return s == 0 && w < l ? w : -1;
    const int rounds = (l + per_xcd - 1) / per_xcd;
    if (s < rounds - 2) return s * per_xcd + w;
    const int b = (rounds - 2) * per_xcd, d = l - b - per_xcd, t = s - (rounds - 2);
    if (w < d) return t == 0 ? b + w : (t == 1 ? b + d + w : -1);
    return t == 0 ? b + 2 * d + (w - d) : -1;
}

// One-item workgroups of the last two rounds over XCDs 0..x-1, and on XCD x
// the first such workgroup (-1 if the list has no such last two rounds).
COC_HD inline int singles_before(const int32_t* tiles_m, int tiles_n, int npieces, int per_xcd, int x,
                                              int* first) {
    int n = 0;
    for (int y = 0; y <= x; ++y) {
        const int l = xcd_items(tiles_m, tiles_n, npieces, y);
        int d = -1, singles = 0;
        if (l > per_xcd) {
            const int rounds = (l + per_xcd - 1) / per_xcd;
            d = l - (rounds - 2) * per_xcd - per_xcd;
            singles = per_xcd - d;
        }
        if (y == x) *first = d;
        else n += singles;
    }
    return n;
}

// The piece holding item j of XCD x's list (npieces if none), and in *jj
// the item's index within that XCD's run of the piece.
COC_HD inline int piece_of_item(const int32_t* tiles_m, int tiles_n, int npieces, int x, int j, int* jj) {
    int c = 0;
    *jj = j;
    for (; c < npieces; ++c) {
        const int t = tiles_m[c] * tiles_n;
        const int cnt = t / 8 + (x < t % 8 ? 1 : 0);
        if (*jj < cnt) break;
        *jj -= cnt;
    }
    return c;
}

// Under schedule_item: one past the last chunk (wait index of a piece; -1:
// none) that the first tile of a two-tile workgroup reads.  Those chunks
// must arrive before the launch's first round can start.
COC_HD inline int early_chunks(const int32_t* tiles, const int32_t* wait, int npieces, int per_xcd) {
    int early = 0;
    for (int x = 0; x < 8; ++x) {
        const int l = xcd_items(tiles, 1, npieces, x);
        for (int w = 0; w < per_xcd; ++w) {
            const int j = schedule_item(l, per_xcd, w, 0);
            if (j < 0 || schedule_item(l, per_xcd, w, 1) < 0) continue;   // one-tile workgroup
            int jj = 0;
            const int c = piece_of_item(tiles, 1, npieces, x, j, &jj);
            if (c < npieces && wait[c] + 1 > early) early = wait[c] + 1;
        }
    }
    return early;
}

// The s-th item of workgroup w in list order: whole rounds w, w + per_xcd,
// ..., so the list's chunks finish in order; -1 past the end.
COC_HD inline int inorder_item(int l, int per_xcd, int w, int s) {
    const int j = w + s * per_xcd;
    return j < l ? j : -1;
}

#endif  // COC_SCHEDULE_H
