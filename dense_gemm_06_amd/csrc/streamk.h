// streamk.h -- the stream-K share of each workgroup of a persistent launch.
//
// "Shared memory and tensor cores" (section 13.10, split-K and stream-K): when the
// output tiles do not divide evenly into the machine's workgroups, the last,
// partial round of tiles leaves most compute units idle. Stream-K instead deals
// the multiply-accumulate iterations (here: k-tiles of 32) of those tiles out
// evenly: the S tail tiles form one linear iteration space of S * KT k-tiles
// (tile by tile, k ascending), and workgroup w of the G that share the tail (G at
// most the grid; fewer spread the tail less and leave fewer partial sums) takes
// the range [bound(w), bound(w + 1)). A range that begins or ends inside a tile leaves a
// partial sum of that tile, which goes to the workspace; a second launch adds the
// partial sums of each split tile in k order (so the result does not depend on
// which workgroup finished first) and writes C.
//
// The equal shares floor(w * S * KT / G) are moved to the nearest tile boundary
// when they fall fewer than 4 k-tiles from it, so that every piece a workgroup
// computes spans at least 4 k-tiles (the copy stream of the persistent kernel runs
// 3 k-tiles ahead and carries over from one piece to the next). With KT >= 8 and
// floor(S * KT / G) >= 4 every non-empty piece then spans at least 4 k-tiles, and
// the bounds stay non-decreasing in w (some shares may become empty).
//
// With fewer tail tiles than workgroups (S < G) a share spans less than one tile
// plus the two moves, so it meets at most two tiles: piece 0 starts at bound(w),
// piece 1 (if any) at the next tile boundary. Workspace slot 2 w + p holds piece
// p's partial sum of workgroup w as a 256 x 256 fp32 tile (row-major, leading
// dimension 256); a piece that covers its whole tile is stored to C directly and
// uses no slot.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "menu.h"

namespace dg {

// floor(a / d) for 0 <= a < 2^53 and 0 < d < 2^31: a 32-bit division when a fits
// in 32 bits, else a double-precision quotient (a and d convert exactly) corrected
// by one step, since the rounded quotient can land on the next integer. A 64-bit
// integer division is a long instruction sequence on the GPU, and the fixup kernel
// takes several of these per tile before its first load.
__host__ __device__ inline int64_t sk_div(int64_t a, int64_t d) {
    if (a < ((int64_t)1 << 32)) return (int64_t)((uint32_t)a / (uint32_t)d);  // the common case
    int64_t q = (int64_t)((double)a / (double)d);
    if (q * d > a) --q;
    else if ((q + 1) * d <= a) ++q;
    return q;
}

// First k-tile (in the tail's linear iteration space of `iters` = S * KT k-tiles)
// of workgroup w's share, w = 0 .. G; bound(0) = 0 and bound(G) = iters.
__host__ __device__ inline int64_t sk_bound(int w, int G, int64_t iters, int KT) {
    int64_t b = sk_div((int64_t)w * iters, G);
    const int64_t r = b - sk_div(b, KT) * KT;
    if (r != 0) {
        if (r < kSkMinPiece) b -= r;
        else if (KT - r < kSkMinPiece) b += KT - r;
    }
    return b;
}

// The largest w in 0 .. G - 1 with sk_bound(w) <= it (bounds are non-decreasing).
// Unmoved bounds are floor(w * iters / G), which puts the owner at floor(it * G /
// iters) give or take the moves; the walks below correct the estimate (a step or
// two: a move is at most 3 k-tiles, a share at least 4).
__host__ __device__ inline int sk_owner(int64_t it, int G, int64_t iters, int KT) {
    int64_t w = sk_div(it * G, iters);
    if (w > G - 1) w = G - 1;
    while (w > 0 && sk_bound((int)w, G, iters, KT) > it) --w;
    while (w + 1 < G && sk_bound((int)w + 1, G, iters, KT) <= it) ++w;
    return (int)w;
}

// Piece p (0 or 1) of workgroup w's share: tail tile `tile` (0 .. S - 1), its first
// k-tile kb and k-tile count nk; false if the share has no such piece.
__host__ __device__ inline bool sk_piece(int w, int p, int G, int S, int KT, int& tile, int& kb, int& nk) {
    const int64_t iters = (int64_t)S * KT;
    const int64_t b0 = sk_bound(w, G, iters, KT), b1 = sk_bound(w + 1, G, iters, KT);
    const int64_t s = p == 0 ? b0 : (sk_div(b0, KT) + 1) * KT;
    if (s >= b1) return false;
    const int64_t t = sk_div(s, KT);
    const int64_t e = b1 < (t + 1) * KT ? b1 : (t + 1) * KT;
    tile = (int)t;
    kb = (int)(s - t * KT);
    nk = (int)(e - s);
    return true;
}

}  // namespace dg
