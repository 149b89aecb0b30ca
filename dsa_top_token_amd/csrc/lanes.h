// Cross-lane exchanges across lane bit 4 (xor 16) and bit 5 (xor 32) on
// VALU permutes instead of LDS round trips (ds_bpermute).
//
// v_permlane16_swap / v_permlane32_swap, given the same register as both
// operands, return the pair {own value, partner's value}: own first in lanes
// whose bit 4 (resp. 5) is 0, partner first in the others.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

__device__ __forceinline__ uint32_t lane_partner16(uint32_t x) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return (threadIdx.x & 16) ? r[0] : r[1];
}

__device__ __forceinline__ uint32_t lane_partner32(uint32_t x) {
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return (threadIdx.x & 32) ? r[0] : r[1];
}

// Maximum / sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48.
__device__ __forceinline__ float lanes4_max(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float lanes4_sum(float v) {
    // {own, partner} in either order: the sum is the same in every lane.
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

}  // namespace dsa
