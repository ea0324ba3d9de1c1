// Device helpers shared by the gfx950 kernels of libgr.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace gr {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float((uint32_t)b << 16);
}

// fp32 -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
    uint32_t u = __float_as_uint(x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}


__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Cross-lane steps on DPP (data-parallel primitives: an operand read from
// another lane of the same 16-lane row, no LDS round trip), for a wavefront
// whose 64 lanes are all active.
//   0xB1 quad_perm [1,0,3,2] (lane ^ 1)    0x4E quad_perm [2,3,0,1] (lane ^ 2)
//   0x111.. row_shr:n   0x124 row_ror:4   0x128 row_ror:8
//   0x142 row_bcast:15 (lane 15 of a row to the next row)
//   0x143 row_bcast:31 (lane 31 to rows 2 and 3)
// A lane with no source (or whose row is masked off) gets `ident`.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v, uint32_t ident) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, CTRL, ROW_MASK, 0xF, false);
}

// AND / OR over all 64 lanes, the same value in every lane: within each
// row by DPP (quad butterflies, then rotations by 4 and 8), then the four
// rows' values by readlane.
__device__ __forceinline__ uint32_t wave_and32(uint32_t x) {
    x &= dpp_u32<0xB1>(x, ~0u);
    x &= dpp_u32<0x4E>(x, ~0u);
    x &= dpp_u32<0x124>(x, ~0u);
    x &= dpp_u32<0x128>(x, ~0u);
    return __builtin_amdgcn_readlane(x, 0) & __builtin_amdgcn_readlane(x, 16) &
           __builtin_amdgcn_readlane(x, 32) & __builtin_amdgcn_readlane(x, 48);
}
__device__ __forceinline__ uint32_t wave_or32(uint32_t x) {
    x |= dpp_u32<0xB1>(x, 0u);
    x |= dpp_u32<0x4E>(x, 0u);
    x |= dpp_u32<0x124>(x, 0u);
    x |= dpp_u32<0x128>(x, 0u);
    return __builtin_amdgcn_readlane(x, 0) | __builtin_amdgcn_readlane(x, 16) |
           __builtin_amdgcn_readlane(x, 32) | __builtin_amdgcn_readlane(x, 48);
}

// Inclusive prefix sum over the 64 lanes: Hillis-Steele shifts by 1, 2, 4, 8
// within each row, then each row adds the totals of the rows before it.
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t x) {
    x += dpp_u32<0x111>(x, 0u);
    x += dpp_u32<0x112>(x, 0u);
    x += dpp_u32<0x114>(x, 0u);
    x += dpp_u32<0x118>(x, 0u);
    x += dpp_u32<0x142, 0xA>(x, 0u);
    x += dpp_u32<0x143, 0xC>(x, 0u);
    return x;
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xF,
                                                      0xF, false));
}

// Max over all 64 lanes (all active), the same value in every lane: the
// 16-lane rows on DPP (lane ^ 1, lane ^ 2, mirror within 8, mirror within
// 16), then the four rows' values by readlane.
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_f32<0xB1>(v));
    v = fmaxf(v, dpp_f32<0x4E>(v));
    v = fmaxf(v, dpp_f32<0x141>(v));
    v = fmaxf(v, dpp_f32<0x140>(v));
    const int b = __float_as_int(v);
    return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 0)),
                       __int_as_float(__builtin_amdgcn_readlane(b, 16))),
                 fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 32)),
                       __int_as_float(__builtin_amdgcn_readlane(b, 48))));
}

// Max / sum over the lane pairs (l, l ^ 16) or (l, l ^ 32) on the gfx950
// row swaps: v_permlane16_swap / v_permlane32_swap hand every lane the
// values of the even and the odd row of its pair, so each lane of the pair
// computes op(even, odd), the same in both.  All lanes active.
__device__ __forceinline__ float pair16_max(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_max(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair16_sum(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair32_sum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Order LDS traffic of one wavefront (lanes exchange data through LDS
// without a workgroup barrier).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Order-preserving map of fp32 onto uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t f32_ord(float f) {
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float f32_unord(uint32_t o) {
    uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
    return __uint_as_float(u);
}

}  // namespace gr
