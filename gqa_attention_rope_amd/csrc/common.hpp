// Device helpers shared by the libgqa kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
// native 16-byte vector (first-class in LLVM, unlike HIP's uint4 struct)
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Cache-policy operand of the raw buffer load/store builtins: the non-temporal
// (streaming) hint, emitted as the "nt" modifier on gfx950.
constexpr int CPOL_NT = 2;

// ---- bf16 <-> fp32 ---------------------------------------------------------

// bf16 in the low / high half of a 32-bit word, widened exactly to fp32
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// the same with the gfx950 conversion instruction (v_cvt_pk_bf16_f32, round to
// nearest even): one instruction for two values
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
    const f32x2_t f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// fp64 -> bf16 rounded once to nearest even.  The value is first narrowed to
// fp32 with round-to-odd (truncate toward zero, then set the last bit when
// anything was dropped); fp32 keeps 16 more bits than bf16, so rounding that
// intermediate to nearest-even gives the correctly rounded bf16 of the fp64
// value (no double-rounding error).
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double x) {
    float f = (float)x;                      // nearest, may be above or below x
    uint32_t u = __float_as_uint(f);
    if ((double)f != x && x == x) {
        if (fabs((double)f) > fabs(x)) u -= 1u;  // step toward zero: truncation
        u |= 1u;                                  // sticky bit
    }
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;  // NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// ---- packed bf16 dot product (v_dot2_f32_bf16) -------------------------------

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                           false);
}

// ---- cross-lane moves ----------------------------------------------------------
// DPP controls (gfx9 encoding): quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E,
// row_half_mirror (lane i <-> 7-i inside 8) = 0x141, row_ror:8 = 0x128.

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}

// v + (v moved by DPP CTRL); bound_ctrl zero-fills lanes without a source, so
// the compiler can fold the move into the add (v_add_f32 with a DPP operand)
template <int CTRL>
__device__ __forceinline__ float add_dpp(float v) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}

// sum over the 8 lanes of each aligned group of 8 (all 8 lanes receive it)
__device__ __forceinline__ float sum8(float v) {
    v = add_dpp<0xB1>(v);
    v = add_dpp<0x4E>(v);
    v = add_dpp<0x141>(v);
    return v;
}

// maximum over lane bits 3, 4 and 5 (the 8 row groups of 8 lanes, values
// replicated inside each group), returned wave-uniform: row_ror:8 pairs the two
// groups of each 16-lane row, row_bcast:15 and row_bcast:31 carry the running
// maximum into rows 1..3, and lane 63 ends up with the maximum of all.
__device__ __forceinline__ float max_rows_uniform(float v) {
    const int ninf = (int)0xff800000u;
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), 0x128, 0xf, 0xf, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), 0x142, 0xa, 0xf, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), 0x143, 0xc, 0xf, false)));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ float xor_f32(float v, int mask) { return __shfl_xor(v, mask, 64); }

// reduce over lane bits 3, 4, 5 (lanes l, l^8, l^16, l^32, ...): 8 values
__device__ __forceinline__ float sum_hi3(float v) {
    v += dpp_f32<0x128>(v);  // row_ror:8 pairs lane i with i^8 inside each row of 16
    v += xor_f32(v, 16);
    v += xor_f32(v, 32);
    return v;
}
__device__ __forceinline__ float max_hi3(float v) {
    v = fmaxf(v, dpp_f32<0x128>(v));
    v = fmaxf(v, xor_f32(v, 16));
    v = fmaxf(v, xor_f32(v, 32));
    return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace gqa
