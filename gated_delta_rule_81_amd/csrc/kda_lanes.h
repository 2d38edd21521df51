// kda_lanes.h -- cross-lane sums and gathers for gfx950 that do not use the
// LDS pipe (permlane swaps and DPP), for the backward and token-recurrence
// kernels.
#pragma once

#include "kda_device.h"

namespace kda {

// Cross-lane sums without the LDS pipe (gfx950 permlane swaps and DPP).
// v_permlane16_swap(a, b) exchanges the odd 16-lane rows of a with the even
// rows of b, v_permlane32_swap(a, b) the upper 32 lanes of a with the lower 32
// of b; with a = b = x the two results add up to x + x[l ^ 16] (x[l ^ 32]).
__device__ __forceinline__ float xor16_sum(float x) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
// Sum over the four lanes l % 16 == const (the four 16-lane rows); every lane
// receives it, added in the same order in all of them.
__device__ __forceinline__ float rows4_sum(float x) { return xor32_sum(xor16_sum(x)); }
// The values of the four lanes l % 16 == const, row by row: v[j] = x of lane
// 16 j + l % 16, in every lane.
__device__ __forceinline__ void rows4_gather(float x, float (&v)[4]) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);  // [r0 r0 r2 r2], [r1 r1 r3 r3]
    const auto e = __builtin_amdgcn_permlane32_swap(p[0], p[0], false, false);  // r0, r2
    const auto o = __builtin_amdgcn_permlane32_swap(p[1], p[1], false, false);  // r1, r3
    v[0] = __uint_as_float(e[0]);
    v[1] = __uint_as_float(o[0]);
    v[2] = __uint_as_float(e[1]);
    v[3] = __uint_as_float(o[1]);
}
// Sum over the 16 lanes of a row, in every lane (DPP row rotations).
template <int N>
__device__ __forceinline__ float dpp_row_ror(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + N, 0xf, 0xf,
                                                      false));
}
__device__ __forceinline__ float row16_total(float x) {
    x += dpp_row_ror<8>(x);
    x += dpp_row_ror<4>(x);
    x += dpp_row_ror<2>(x);
    x += dpp_row_ror<1>(x);
    return x;
}

}  // namespace kda
