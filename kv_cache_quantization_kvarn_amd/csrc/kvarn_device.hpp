// Device helpers for the KVarN kernels on gfx950 (CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvarn {

// Workgroup and work-item indices read straight from the hardware registers.
// The blockIdx / threadIdx accessors go through device-library functions
// built with IEEE mode on; kernels built with it off cannot inline them, so
// each use becomes a call whose entry waits for every memory operation in
// flight.  The quantize kernel reads its indices here (1-3 % faster on four
// of the five benchmark layers, the fifth unchanged); the decode kernels keep
// the accessors, whose calls sit in their prologues only (the call-free form
// of those measured 1-2 % slower).
__device__ __forceinline__ unsigned wg_x() { return __builtin_amdgcn_workgroup_id_x(); }
__device__ __forceinline__ unsigned wg_y() { return __builtin_amdgcn_workgroup_id_y(); }
__device__ __forceinline__ unsigned wg_z() { return __builtin_amdgcn_workgroup_id_z(); }
__device__ __forceinline__ unsigned tid_x() { return __builtin_amdgcn_workitem_id_x(); }

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

// Reductions over the 64 lanes, every lane ending with the result, entirely
// on the VALU: DPP inside each 16-lane row (xor 1, xor 2, then rotations by 4
// and 8), then v_permlane16_swap and v_permlane32_swap, each of which, given
// the same value twice, returns the halves whose combination is v op v[l ^ 16]
// (resp. v[l ^ 32]).
__device__ __forceinline__ float wave_max_all(float v) {
    v = fmaxf(v, i2f(__builtin_amdgcn_mov_dpp(f2i(v), 0xB1, 0xF, 0xF, false)));   // quad_perm xor 1
    v = fmaxf(v, i2f(__builtin_amdgcn_mov_dpp(f2i(v), 0x4E, 0xF, 0xF, false)));   // quad_perm xor 2
    v = fmaxf(v, i2f(__builtin_amdgcn_mov_dpp(f2i(v), 0x124, 0xF, 0xF, false)));  // row_ror 4
    v = fmaxf(v, i2f(__builtin_amdgcn_mov_dpp(f2i(v), 0x128, 0xF, 0xF, false)));  // row_ror 8
    const auto a16 = __builtin_amdgcn_permlane16_swap((unsigned)f2i(v), (unsigned)f2i(v), false, false);
    v = fmaxf(i2f((int)a16[0]), i2f((int)a16[1]));
    const auto a32 = __builtin_amdgcn_permlane32_swap((unsigned)f2i(v), (unsigned)f2i(v), false, false);
    return fmaxf(i2f((int)a32[0]), i2f((int)a32[1]));
}

__device__ __forceinline__ float wave_sum_all(float v) {
    v += i2f(__builtin_amdgcn_update_dpp(0, f2i(v), 0xB1, 0xF, 0xF, true));
    v += i2f(__builtin_amdgcn_update_dpp(0, f2i(v), 0x4E, 0xF, 0xF, true));
    v += i2f(__builtin_amdgcn_update_dpp(0, f2i(v), 0x124, 0xF, 0xF, true));
    v += i2f(__builtin_amdgcn_update_dpp(0, f2i(v), 0x128, 0xF, 0xF, true));
    const auto a16 = __builtin_amdgcn_permlane16_swap((unsigned)f2i(v), (unsigned)f2i(v), false, false);
    v = i2f((int)a16[0]) + i2f((int)a16[1]);
    const auto a32 = __builtin_amdgcn_permlane32_swap((unsigned)f2i(v), (unsigned)f2i(v), false, false);
    return i2f((int)a32[0]) + i2f((int)a32[1]);
}

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

__device__ __forceinline__ uint32_t float_to_half_bits(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// x, rounded to fp32, as a value the compiler cannot see through: an fp16
// conversion of it is not fused with the product that made it.  (A fused
// v_fma_mix rounds the exact product to fp16 once, a conversion of the fp32
// product rounds twice; the two differ by one fp16 ulp where the fp32
// product lands on an fp16 tie, so a value split into fp16 high and low
// parts must take both parts, at every use, from the same fp32 number.)
__device__ __forceinline__ float fp32_value(float x) {
    asm("" : "+v"(x));
    return x;
}


// Query elements of the three query dtypes of the C ABI (0 float32, 1
// float16, 2 bfloat16), widened exactly to float.
__device__ __forceinline__ float q_at(const void* q, int dt, int64_t idx) {
    if (dt == 0) return static_cast<const float*>(q)[idx];
    const uint32_t h = static_cast<const uint16_t*>(q)[idx];
    return dt == 2 ? __builtin_bit_cast(float, h << 16) : half_bits_to_float(h);
}
// N = 4 or 8 consecutive elements from idx, a multiple of N (whole 8- or
// 16-byte units for the 16-bit dtypes)
template <int N>
__device__ __forceinline__ void q_load(const void* q, int dt, int64_t idx, float (&x)[N]) {
    static_assert(N == 4 || N == 8, "4 or 8 elements");
    if (dt == 0) {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(q) + idx);
#pragma unroll
        for (int k = 0; k < N / 4; k++) {
            const float4 v = p[k];
            x[4 * k] = v.x; x[4 * k + 1] = v.y; x[4 * k + 2] = v.z; x[4 * k + 3] = v.w;
        }
        return;
    }
    uint32_t w[N / 2];
    if constexpr (N == 8) {
        const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(q) + idx);
        w[0] = u.x; w[1] = u.y; w[2] = u.z; w[3] = u.w;
    } else {
        const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(q) + idx);
        w[0] = u.x; w[1] = u.y;
    }
#pragma unroll
    for (int k = 0; k < N / 2; k++) {
        if (dt == 2) {
            x[2 * k] = __builtin_bit_cast(float, w[k] << 16);
            x[2 * k + 1] = __builtin_bit_cast(float, w[k] & 0xffff0000u);
        } else {
            x[2 * k] = half_bits_to_float(w[k] & 0xffffu);
            x[2 * k + 1] = half_bits_to_float(w[k] >> 16);
        }
    }
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// LDS-DMA loads: each active lane's 16 bytes at buffer offset voff + soff
// land at LDS address lds + 16 lane.  Written as instructions so
// that the compiler's wait-count tracking, which would hold every later LDS
// read until all such loads have landed, stays out of the way: the caller
// waits with s_waitcnt vmcnt before reading the bytes and keeps no other
// vector-memory load in flight across them.  M0 carries the LDS address (the
// compiler keeps nothing in M0 in these kernels).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// lds and soff must be wave-uniform.
__device__ __forceinline__ void lds_dma16(uint32_t lds, i32x4 rsrc, uint32_t voff, int soff) {
    lds = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds);
    soff = __builtin_amdgcn_readfirstlane(soff);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 ::"s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
}
// Two such loads with one M0: the second one's 16 bytes land 1024 bytes
// further on in LDS, and its instruction offset of 1024 is added to both of
// its addresses, so voff1 is its byte offset less 1024 (voff1 + 1024 >= 1024).
__device__ __forceinline__ void lds_dma16x2(uint32_t lds, i32x4 rsrc, uint32_t voff0, uint32_t voff1, int soff) {
    lds = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds);
    soff = __builtin_amdgcn_readfirstlane(soff);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %3, %4 offen lds\n\t"
                 "buffer_load_dwordx4 %2, %3, %4 offen offset:1024 lds"
                 ::"s"(lds), "v"(voff0), "v"(voff1), "s"(rsrc), "s"(soff) : "memory", "m0");
}
// N (1, 2 or 4) such loads with one M0 and one lane offset: load i reads the
// memory 1024 i bytes after load 0's and lands 1024 i bytes after it in LDS.
template <int N>
__device__ __forceinline__ void lds_dma16_run(uint32_t lds, i32x4 rsrc, uint32_t voff, int soff) {
    static_assert(N == 1 || N == 2 || N == 4, "runs of 1, 2 or 4 KB");
    lds = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds);
    soff = __builtin_amdgcn_readfirstlane(soff);
    if constexpr (N == 1) {
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                     ::"s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
    } else if constexpr (N == 2) {
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds\n\t"
                     "buffer_load_dwordx4 %1, %2, %3 offen offset:1024 lds"
                     ::"s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
    } else {
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds\n\t"
                     "buffer_load_dwordx4 %1, %2, %3 offen offset:1024 lds\n\t"
                     "buffer_load_dwordx4 %1, %2, %3 offen offset:2048 lds\n\t"
                     "buffer_load_dwordx4 %1, %2, %3 offen offset:3072 lds"
                     ::"s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
    }
}
// N KB (N = 1 .. 8 but 3, 5, 7) as runs of at most 4 (the instruction offset
// stops at 4095)
template <int N>
__device__ __forceinline__ void lds_dma16_runs(uint32_t lds, i32x4 rsrc, uint32_t voff, int soff) {
    if constexpr (N <= 4) {
        lds_dma16_run<N>(lds, rsrc, voff, soff);
    } else {
        lds_dma16_run<4>(lds, rsrc, voff, soff);
        lds_dma16_run<N - 4>(lds + 4096u, rsrc, voff + 4096u, soff);
    }
}
#pragma clang diagnostic pop
// LDS byte address of a pointer into __shared__ memory
__device__ __forceinline__ uint32_t lds_address(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// raw buffer resource over [base, base + bytes): 32-bit offsets, no stride
__device__ __forceinline__ i32x4 raw_buffer(const void* base, uint32_t bytes) {
    const uint64_t p = (uint64_t)(uintptr_t)base;
    return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)p), __builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32)),
               __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000};
}

}  // namespace kvarn
