// Device helpers shared by the libspark kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define SPARK_WAVE 64

namespace spark {

// bf16 bits -> fp32 (exact widening).
__device__ __forceinline__ float bf16_lo(uint32_t two) { return __uint_as_float(two << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t two) { return __uint_as_float(two & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

__device__ __forceinline__ uint32_t lane_id() { return __lane_id(); }

// 64-bit lane mask of lanes whose predicate holds.
__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Number of set bits of m below this lane (v_mbcnt_lo / v_mbcnt_hi).
__device__ __forceinline__ uint32_t mbcnt(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Wave-wide reductions over 64 lanes (butterfly through ds_swizzle / DPP as the compiler picks).
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

// Wave-wide max through DPP (no LDS traffic): butterfly inside each 16-lane
// row, then the four row results combined from lanes 0, 16, 32, 48. The DPP
// steps are moves with no old value, which the compiler folds into the max
// or add that uses them; these patterns never read outside a row, so the
// bound control setting does not apply.
__device__ __forceinline__ float dpp_row_max(float x) {
    int v = __float_as_int(x);
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true)));  // quad_perm 1,0,3,2
    v = __float_as_int(x);
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true)));  // quad_perm 2,3,0,1
    v = __float_as_int(x);
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, true))); // row_half_mirror
    v = __float_as_int(x);
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, true))); // row_mirror
    return x;
}
__device__ __forceinline__ float wave_max_dpp(float x) {
    x = dpp_row_max(x);
    const int v = __float_as_int(x);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(v, 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(v, 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(v, 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(v, 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Sum of x over lanes L and L^16 (then L^32): the two outputs of a gfx950
// permlane swap hold this lane's value and its partner's, in either order.
__device__ __forceinline__ float xor16_sum(float x) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Wave-wide sum without LDS: DPP butterfly inside each 16-lane row, then the
// rows combined with permlane swaps. Every lane gets the total.
__device__ __forceinline__ float wave_sum_dpp(float x) {
    int v = __float_as_int(x);
    x += __int_as_float(__builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true));   // quad_perm 1,0,3,2
    v = __float_as_int(x);
    x += __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true));   // quad_perm 2,3,0,1
    v = __float_as_int(x);
    x += __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, true));  // row_half_mirror
    v = __float_as_int(x);
    x += __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, true));  // row_mirror
    return xor32_sum(xor16_sum(x));
}

// LDS written by some lanes of a wave and read by others: order the accesses
// within the wave (no workgroup barrier needed).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

}  // namespace spark
