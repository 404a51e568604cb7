// Device helpers for the KVarN kernels on gfx950 (CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvarn {

__device__ __forceinline__ int f2i(float v) { return __builtin_bit_cast(int, v); }
__device__ __forceinline__ float i2f(int v) { return __builtin_bit_cast(float, v); }

// v of the lane whose index differs in bit BIT (0..4).  Bits 0, 1 and 3 use
// DPP (quad_perm for 1 and 2, row_ror:8 inside a 16-lane row for 8); bits 2
// and 4 use ds_swizzle in bitmask mode (xor mask 4 or 16).
template <int BIT>
__device__ __forceinline__ float xor_lane(float v) {
    static_assert(BIT >= 0 && BIT <= 4, "lane bit");
    if constexpr (BIT == 0) {
        return i2f(__builtin_amdgcn_mov_dpp(f2i(v), 0xB1, 0xF, 0xF, false));
    } else if constexpr (BIT == 1) {
        return i2f(__builtin_amdgcn_mov_dpp(f2i(v), 0x4E, 0xF, 0xF, false));
    } else if constexpr (BIT == 3) {
        return i2f(__builtin_amdgcn_mov_dpp(f2i(v), 0x128, 0xF, 0xF, false));
    } else if constexpr (BIT == 2) {
        return i2f(__builtin_amdgcn_ds_swizzle(f2i(v), 0x101F));
    } else {
        return i2f(__builtin_amdgcn_ds_swizzle(f2i(v), 0x401F));
    }
}

__device__ __forceinline__ float lane_bcast32(float v) {
    // value of lane (l ^ 32)
    return i2f(__builtin_amdgcn_ds_bpermute(((int)(threadIdx.x & 63) ^ 32) << 2, f2i(v)));
}

__device__ __forceinline__ float wave_max_all(float v) {
    v = fmaxf(v, xor_lane<0>(v));
    v = fmaxf(v, xor_lane<1>(v));
    v = fmaxf(v, xor_lane<2>(v));
    v = fmaxf(v, xor_lane<3>(v));
    v = fmaxf(v, xor_lane<4>(v));
    v = fmaxf(v, lane_bcast32(v));
    return v;
}

__device__ __forceinline__ float wave_sum_all(float v) {
    v += xor_lane<0>(v);
    v += xor_lane<1>(v);
    v += xor_lane<2>(v);
    v += xor_lane<3>(v);
    v += xor_lane<4>(v);
    v += lane_bcast32(v);
    return v;
}

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

__device__ __forceinline__ uint32_t float_to_half_bits(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

}  // namespace kvarn
