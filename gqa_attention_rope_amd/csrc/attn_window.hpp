// Tile geometry of a decode query under an optional sliding window with
// attention sinks ([P7] "Part 7: The Modern Decoder Block", modules L7.5 and
// L7.7 name the window and the sinks; the query at position L - 1 sees rows
// L - window .. L - 1 and rows 0 .. n_sink - 1).
#pragma once

#include <hip/hip_runtime.h>

namespace gqa {

// Visible rows of the new query of a sequence with L = past_len + 1 cached
// rows: all of them, or, under a sliding window of W rows, the sink rows
// 0 .. n_sink-1 and the window rows w0 .. L-1 with w0 = L - W.  The 64-row tiles of
// the segment are the nst sink tiles 0 .. nst-1 followed by the window tiles
// at0, at0+1, .. (absolute 64-row tile indices); when the two ranges meet
// (or there is no window) the tiles are simply 0 .. ceil(L/64)-1 and w0 = 0.
struct Geo {
    int nt;   // tiles of the segment
    int nst;  // leading tiles (sinks, or all of them when contiguous)
    int at0;  // absolute index of the first window tile
    int w0;   // first visible window row (0 when every row is visible)
};
__device__ __forceinline__ Geo geo_of(int L, int window, int n_sink) {
    Geo g;
    const int all = (L + 63) / 64;
    if (window <= 0 || L - window <= n_sink) {
        g.nt = all;
        g.nst = all;
        g.at0 = all;
        g.w0 = 0;
    } else {
        g.w0 = L - window;
        g.nst = (n_sink + 63) / 64;
        const int a0 = g.w0 / 64;
        g.at0 = a0 > g.nst ? a0 : g.nst;
        g.nt = g.nst + all - g.at0;
    }
    return g;
}

}  // namespace gqa
