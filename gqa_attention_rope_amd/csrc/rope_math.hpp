// RoPE arithmetic shared by the kernels that rotate q and k (fp64 angles,
// one rounding to bf16 per output).
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace gqa {

// (a, b) -> (a cos - b sin, a sin + b cos), fp64, each output rounded once to bf16.
__device__ __forceinline__ void turn(float a, float b, double c, double s, uint32_t& ra, uint32_t& rb) {
    double da = (double)a, db = (double)b;
    ra = f64_to_bf16_rne(da * c - db * s);
    rb = f64_to_bf16_rne(da * s + db * c);
}

// Rotate item c of a head: 8 pairs held as two 16-byte pieces w[0..3] and
// w[4..7].  Interleaved layout: word m holds pair 8c + m as (lo, hi) = (a, b).
// Half layout: value m of the first piece pairs with value m of the second
// (pair 8c + m).  cs / sn hold the (scaled) cos / sin of every pair.
__device__ __forceinline__ void rotate_item(const uint32_t (&w)[8], int c, int layout, const double* cs,
                                            const double* sn, uint32_t (&o)[8]) {
    if (layout == 0) {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int i = 8 * c + m;
            uint32_t ra, rb;
            turn(bf_lo(w[m]), bf_hi(w[m]), cs[i], sn[i], ra, rb);
            o[m] = ra | (rb << 16);
        }
    } else {
#pragma unroll
        for (int m = 0; m < 8; m += 2) {
            const int i = 8 * c + m;
            uint32_t ra0, rb0, ra1, rb1;
            turn(bf_lo(w[m / 2]), bf_lo(w[4 + m / 2]), cs[i], sn[i], ra0, rb0);
            turn(bf_hi(w[m / 2]), bf_hi(w[4 + m / 2]), cs[i + 1], sn[i + 1], ra1, rb1);
            o[m / 2] = ra0 | (ra1 << 16);
            o[4 + m / 2] = rb0 | (rb1 << 16);
        }
    }
}

}  // namespace gqa
