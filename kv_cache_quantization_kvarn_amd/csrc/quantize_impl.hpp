// KVarN quantize kernel for gfx950 (templates; instantiated per head_dim in
// quantize_d128.hip, quantize_d256.hip and quantize_d512.hip).
//
// One workgroup turns one fp16 tile (T tokens x D channels of one KV head)
// into one record: Hadamard rotation across channels, column/row
// normalization iterations, per-token asymmetric round-to-nearest, packed
// codes (evermx.com KVarN review, method paragraph: the four stages; gmlx
// "KV cache quantization", "The two schemes": per-head Hadamard rotation,
// records scaled so that no token or channel dominates).
//
// Register layout: every lane holds R = 4 consecutive tokens x C = 16
// consecutive channels (64 values).  D/16 lanes share a token row; their
// lane-index bits carry the channel group and are chosen among bits 0, 1, 3
// (DPP patterns: quad_perm and row_ror:8), then 2 and 4 (ds_swizzle).  The
// remaining lane bits (of 2, 4, 5) and the wave index carry the row group.
//
// The rotation is the unnormalized +-1 butterfly (4 in-lane stages, then one
// cross-lane stage per channel-group bit).  Statistics use the squared tile
// A = y^2; with a_i = exp(-2 lr_i) and b_j = exp(-2 lc_j), the column step
// is b_j = T / sum_i A_ij a_i and the row step a_i = D / sum_j A_ij b_j --
// the log-space updates "lc_j += ln sigma_j", "lr_i += ln sigma_i" with the
// root-mean-square sigma, written multiplicatively.  A zero or non-finite
// sum leaves the scale unchanged.  The last row step is skipped: the row
// scale multiplies a token's range and minimum alike and cancels from every
// stored value.
#pragma once

#include "kvarn_device.hpp"
#include "kvarn_internal.hpp"

namespace kvarn {
namespace {

constexpr int QC = 16;  // channels per lane
constexpr int QR = 4;   // rows per lane
// x + kMagic (1.5 * 2^23) rounds x half-to-even to an integer kept in the low
// mantissa bits, for -0.5 <= x < 2^22; bits 22 and up hold the constant.
constexpr float kMagic = 12582912.0f;

// lane bit carrying channel-group bit k
__device__ __forceinline__ constexpr int cg_lane_bit(int k) {
    return k == 0 ? 0 : k == 1 ? 1 : k == 2 ? 3 : k == 3 ? 2 : 4;
}

// v + v[lane ^ (1 << BIT)]: one fused v_add_f32_dpp for bits 0, 1, 3.
template <int BIT>
__device__ __forceinline__ float xsum(float v) {
    if constexpr (BIT == 0) return v + i2f(__builtin_amdgcn_update_dpp(0, f2i(v), 0xB1, 0xF, 0xF, true));
    else if constexpr (BIT == 1) return v + i2f(__builtin_amdgcn_update_dpp(0, f2i(v), 0x4E, 0xF, 0xF, true));
    else if constexpr (BIT == 3) return v + i2f(__builtin_amdgcn_update_dpp(0, f2i(v), 0x128, 0xF, 0xF, true));
    else return v + xor_lane<BIT>(v);
}

template <int CGB>
__device__ __forceinline__ float row_sum(float v) {
    v = xsum<0>(v);
    v = xsum<1>(v);
    v = xsum<3>(v);
    if constexpr (CGB >= 4) v = xsum<2>(v);
    if constexpr (CGB >= 5) v = xsum<4>(v);
    return v;
}

template <int CGB>
__device__ __forceinline__ void row_minmax(float& mn, float& mx) {
    mn = fminf(mn, xor_lane<0>(mn)); mx = fmaxf(mx, xor_lane<0>(mx));
    mn = fminf(mn, xor_lane<1>(mn)); mx = fmaxf(mx, xor_lane<1>(mx));
    mn = fminf(mn, xor_lane<3>(mn)); mx = fmaxf(mx, xor_lane<3>(mx));
    if constexpr (CGB >= 4) { mn = fminf(mn, xor_lane<2>(mn)); mx = fmaxf(mx, xor_lane<2>(mx)); }
    if constexpr (CGB >= 5) { mn = fminf(mn, xor_lane<4>(mn)); mx = fmaxf(mx, xor_lane<4>(mx)); }
}

// Cross-lane butterfly on lane bit BIT for 16 values: v <- v + s * partner,
// s = +1 where the bit is clear and -1 where it is set, i.e. (l, u) ->
// (l + u, u - l).  The upper output is the negated butterfly difference;
// the negations commute with the other stages and leave every channel
// multiplied by (-1)^(number of its cross-lane bits), undone at the end.
// Bits 0, 1, 3: one v_fmac_f32_dpp each.
#define KVARN_FMAC_DPP8(CTRL)                                                                   \
    asm volatile("s_nop 1\n\t"                                                                   \
                 "v_fmac_f32_dpp %0, %0, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"             \
                 "v_fmac_f32_dpp %1, %1, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"             \
                 "v_fmac_f32_dpp %2, %2, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"             \
                 "v_fmac_f32_dpp %3, %3, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"             \
                 "v_fmac_f32_dpp %4, %4, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"             \
                 "v_fmac_f32_dpp %5, %5, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"             \
                 "v_fmac_f32_dpp %6, %6, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"             \
                 "v_fmac_f32_dpp %7, %7, %8 " CTRL " row_mask:0xf bank_mask:0xf"                 \
                 : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]),       \
                   "+v"(v[6]), "+v"(v[7])                                                         \
                 : "v"(s))

template <int BIT>
__device__ __forceinline__ void xbutterfly8(float* v, float s) {
    if constexpr (BIT == 0) {
        KVARN_FMAC_DPP8("quad_perm:[1,0,3,2]");
    } else if constexpr (BIT == 1) {
        KVARN_FMAC_DPP8("quad_perm:[2,3,0,1]");
    } else if constexpr (BIT == 3) {
        KVARN_FMAC_DPP8("row_ror:8");
    } else {
#pragma unroll
        for (int k = 0; k < 8; k++) v[k] = fmaf(xor_lane<BIT>(v[k]), s, v[k]);
    }
}

template <int BIT>
__device__ __forceinline__ void xbutterfly(float (&y)[QR][QC], int lane) {
    const float s = ((lane >> BIT) & 1) ? -1.f : 1.f;
#pragma unroll
    for (int r = 0; r < QR; r++) {
        xbutterfly8<BIT>(&y[r][0], s);
        xbutterfly8<BIT>(&y[r][8], s);
    }
}

__device__ __forceinline__ bool usable(float s) { return s > 0.f && s <= 3.0e38f; }

__device__ __forceinline__ uint32_t fbits(float x) { return __builtin_bit_cast(uint32_t, x); }

// Codes sit in the low bits of magic-rounded floats (junk from bit 22 up).
// Pack n consecutive codes of width B into the low n*B bits; n*B <= 16 keeps
// the junk of every addend above the result.
template <int B>
__device__ __forceinline__ uint32_t pack2(uint32_t f0, uint32_t f1) {  // low 2B bits clean
    return (f1 << B) + f0;
}

__device__ __forceinline__ uint32_t bytes4(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3) {
    // byte 0 of each argument -> one dword
    const uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);
    const uint32_t hi = __builtin_amdgcn_perm(b3, b2, 0x0c0c0400u);
    return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// 4 codes of 6 bits -> low 24 bits (clean above).
__device__ __forceinline__ uint32_t pack6x4(uint32_t f0, uint32_t f1, uint32_t f2, uint32_t f3) {
    const uint32_t x01 = ((f1 << 6) + f0) & 0xfffu;
    const uint32_t x23 = (f3 << 6) + f2;   // bits 12..27 zero, junk from 28
    return (x23 << 12) | x01;              // junk shifted out
}

// D = 128: the rotation runs on the 16x16x32 fp16 MFMA (y = X H with the
// fp16 tile as the A operand and +-1 blocks of H as the B operand), each wave
// on its own 32 rows, and reaches the register layout through LDS.
template <int D>
struct MfmaRotation {
    static constexpr bool on = D == 128;
};

// LDS unit (4 floats) of rotated column j (0..63 of the half being moved),
// rows 4 ru .. 4 ru + 3 of a wave's 32 rows: column-major with the row unit
// xor-ed with column bits, so that the MFMA-layout stores and the
// register-layout loads each touch every bank once.
__device__ __forceinline__ int rot_unit(int j, int ru) {
    return 8 * j + (ru ^ ((j ^ (j >> 3)) & 7));
}

template <int D, int T>
struct TileShape {
    static constexpr int LPR = D / QC;                        // lanes per token row
    static constexpr int CGB = LPR == 8 ? 3 : LPR == 16 ? 4 : 5;
    static constexpr int RGB = 6 - CGB;                       // row-group bits inside a wave
    static constexpr int RPW = QR << RGB;                     // rows per wave
    static constexpr int NW = T / RPW;                        // waves per workgroup
    static constexpr int NT = NW * 64;
    static constexpr int NSUB = (RGB == 3) ? 2 : 1;           // lane bit 2 left after the swaps
    static constexpr int SMEM_CODES = T * D;                  // one byte per code at most
    static constexpr int SMEM_PART = NW * NSUB * D * 4;
    static constexpr int SMEM_ROT = MfmaRotation<D>::on ? T * D * 2 : 0;  // half the rotated tile, fp32
    static constexpr int SMEM_A = SMEM_CODES > SMEM_PART ? SMEM_CODES : SMEM_PART;
    // with the MFMA rotation the column partials get their own region after
    // the tile image, so the statistics need not wait for the image to die
    static constexpr int PART_OFF = MfmaRotation<D>::on ? (SMEM_ROT > SMEM_CODES ? SMEM_ROT : SMEM_CODES) : 0;
    static constexpr int SMEM = MfmaRotation<D>::on ? PART_OFF + SMEM_PART : (SMEM_A > SMEM_ROT ? SMEM_A : SMEM_ROT);
};

// One tile -> one record.  smem: TileShape::SMEM bytes; vec: 3*D floats.
template <int D, int T, int BITS, bool CHMAJOR>
__device__ __forceinline__ void quantize_tile(const uint16_t* __restrict__ tile, uint8_t* __restrict__ rec,
                                              uint8_t* smem, float* vec, int32_t n_iters) {
    using S = TileShape<D, T>;
    constexpr int CGB = S::CGB, RGB = S::RGB, RPW = S::RPW, NW = S::NW, NT = S::NT, NSUB = S::NSUB;
    constexpr int QMAX = (1 << BITS) - 1;
    constexpr int CODE_BYTES = T * D * BITS / 8;
    constexpr int REC = CODE_BYTES + 4 * T + 2 * D;
    constexpr int NPART = (RGB >= 2) ? 4 : 8;          // column partials per lane after swaps
    constexpr bool KEEP_Y = D <= 256;                  // D = 512 rebuilds y from y^2 and signs
    static_assert(T * D / 64 == NT, "one lane per 64 values");
    static_assert(REC % 16 == 0, "records stay 16-byte aligned");

    float* colpart = reinterpret_cast<float*>(smem + S::PART_OFF);
    float* bvec = vec;           // b_j = exp(-2 lc_j), unnormalized basis
    float* icvec = vec + D;      // (+-1 per channel) * sqrt(b_j): multiplies y into W
    uint16_t* cvec = reinterpret_cast<uint16_t*>(vec + 2 * D);  // fp16 column scales

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    int cg = 0;
#pragma unroll
    for (int k = 0; k < CGB; k++) cg |= ((lane >> cg_lane_bit(k)) & 1) << k;
    int rg = 0;
    if constexpr (RGB == 3) rg = ((lane >> 2) & 1) | (((lane >> 4) & 1) << 1) | (((lane >> 5) & 1) << 2);
    if constexpr (RGB == 2) rg = ((lane >> 4) & 1) | (((lane >> 5) & 1) << 1);
    if constexpr (RGB == 1) rg = (lane >> 5) & 1;
    const int row0 = wave * RPW + rg * QR;
    const int ch0 = cg * QC;

    float y[QR][QC];
    if constexpr (MfmaRotation<D>::on) {
        // ---- stages 1-2: y = X H on the MFMA, then into the register layout ----
        // H_128 = H_4 (x) H_32 over channel j = 32 v + u: the MFMA takes each
        // 32-channel group v through H_32 (k = u = 8 g4 + i, n = u' = 16 nb + l16,
        // H_32[u][u'] = (-1)^popcount(i & l16 & 7) (-1)^(g4_0 l16_3) (-1)^(g4_1 nb):
        // one per-lane pattern per nb), and the 4 groups meet in an in-lane
        // 4-point butterfly.
        typedef _Float16 h8 __attribute__((ext_vector_type(8)));
        typedef float f4 __attribute__((ext_vector_type(4)));
        static_assert(RGB == 3 && CGB == 3 && RPW == 32, "rotation layout assumes 32 rows x 128 channels per wave");
        const int l16 = lane & 15, g4 = lane >> 4;
        // bit i of wm is parity(i & l16 & 7) (a row of the 8x8 Hadamard matrix)
        const uint32_t m7 = (uint32_t)(l16 & 7);
        const uint32_t wm = ((m7 & 1u) ? 0xAAu : 0u) ^ ((m7 & 2u) ? 0xCCu : 0u) ^ ((m7 & 4u) ? 0xF0u : 0u);
        h8 hp[2];
#pragma unroll
        for (int nb = 0; nb < 2; nb++) {
            const uint32_t flip = ((g4 & 1) & (l16 >> 3)) ^ ((g4 >> 1) & nb);
            const uint32_t sw = wm ^ (flip ? 0xFFu : 0u);
            uint32_t d[4];
#pragma unroll
            for (int k = 0; k < 4; k++) d[k] = 0x3C003C00u | (((sw >> (2 * k)) & 1u) << 15) | (((sw >> (2 * k + 1)) & 1u) << 31);
            hp[nb] = __builtin_bit_cast(h8, make_uint4(d[0], d[1], d[2], d[3]));
        }
        // the wave's 32 x 128 block moves in two halves of 64 columns; lanes
        // whose 16 channels lie in the half read it
        // the wave's 32 x 128 block moves in two halves of 64 columns; lanes
        // whose 16 channels lie in the half read it
        float* yt = reinterpret_cast<float*>(smem) + wave * (RPW * D / 2);
        f4 z[2][4][2];  // [token block][channel group v][nb]
#pragma unroll
        for (int tb = 0; tb < 2; tb++) {
            const uint16_t* xr = tile + (int64_t)(wave * RPW + 16 * tb + l16) * D + 8 * g4;
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const h8 xa = *reinterpret_cast<const h8*>(xr + 32 * v);
#pragma unroll
                for (int nb = 0; nb < 2; nb++)
                    z[tb][v][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa, hp[nb], f4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            }
        }
        // H_4 across the groups: z[.][v'][.] becomes output group v'
#pragma unroll
        for (int tb = 0; tb < 2; tb++)
#pragma unroll
            for (int nb = 0; nb < 2; nb++) {
                const f4 a0 = z[tb][0][nb] + z[tb][1][nb], a1 = z[tb][0][nb] - z[tb][1][nb];
                const f4 a2 = z[tb][2][nb] + z[tb][3][nb], a3 = z[tb][2][nb] - z[tb][3][nb];
                z[tb][0][nb] = a0 + a2;
                z[tb][1][nb] = a1 + a3;
                z[tb][2][nb] = a0 - a2;
                z[tb][3][nb] = a1 - a3;
            }
#pragma unroll
        for (int half = 0; half < 2; half++) {
            // output columns 32 v + 16 nb + l16 with v = 2 half + (0, 1)
#pragma unroll
            for (int tb = 0; tb < 2; tb++)
#pragma unroll
                for (int vq = 0; vq < 2; vq++)
#pragma unroll
                    for (int nb = 0; nb < 2; nb++)
                        *reinterpret_cast<f4*>(yt + 4 * rot_unit(32 * vq + 16 * nb + l16, 4 * tb + g4)) = z[tb][2 * half + vq][nb];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            if ((cg >> 2) == half) {
#pragma unroll
                for (int c = 0; c < QC; c++) {
                    const f4 v = *reinterpret_cast<const f4*>(yt + 4 * rot_unit((ch0 & 63) + c, rg));
#pragma unroll
                    for (int r = 0; r < QR; r++) y[r][c] = v[r];
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
        if (tid < D) bvec[tid] = 1.0f / (float)D;  // c_j = 1 in the normalized basis
    } else {
        // ---- stage 1: load the fp16 tile ---------------------------------------
#pragma unroll
        for (int r = 0; r < QR; r++) {
            const uint4* p = reinterpret_cast<const uint4*>(tile + (int64_t)(row0 + r) * D + ch0);
            uint4 u0 = p[0], u1 = p[1];
            uint32_t w[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
            for (int k = 0; k < 8; k++) {
                y[r][2 * k] = half_bits_to_float(w[k] & 0xffffu);
                y[r][2 * k + 1] = half_bits_to_float(w[k] >> 16);
            }
        }
        if (tid < D) bvec[tid] = 1.0f / (float)D;  // c_j = 1 in the normalized basis

        // ---- stage 2: Hadamard rotation (unnormalized butterflies) -------------
#pragma unroll
        for (int r = 0; r < QR; r++) {
#pragma unroll
            for (int hs = 1; hs < QC; hs <<= 1) {
#pragma unroll
                for (int c = 0; c < QC; c++) {
                    if ((c & hs) == 0) {
                        float a = y[r][c], b = y[r][c + hs];
                        y[r][c] = a + b;
                        y[r][c + hs] = a - b;
                    }
                }
            }
        }
        xbutterfly<0>(y, lane);
        xbutterfly<1>(y, lane);
        xbutterfly<3>(y, lane);
        if constexpr (CGB >= 4) xbutterfly<2>(y, lane);
        if constexpr (CGB >= 5) xbutterfly<4>(y, lane);
    }

    // ---- stage 3: normalization iterations on A = y^2 ----------------------
    float A[QR][QC];
    uint32_t negbits[QR] = {0, 0, 0, 0};
#pragma unroll
    for (int r = 0; r < QR; r++)
#pragma unroll
        for (int c = 0; c < QC; c++) {
            A[r][c] = y[r][c] * y[r][c];
            if constexpr (!KEEP_Y) negbits[r] |= (y[r][c] < 0.f ? 1u : 0u) << c;
        }

    float aw[QR] = {1.f, 1.f, 1.f, 1.f};
    float bw[QC];
    for (int it = 0; it < n_iters; it++) {
        const bool last = it == n_iters - 1;
        // column step: partial sums over this lane's rows
        float p[QC];
#pragma unroll
        for (int c = 0; c < QC; c++) {
            float s = A[0][c] * aw[0];
#pragma unroll
            for (int r = 1; r < QR; r++) s = fmaf(A[r][c], aw[r], s);
            p[c] = s;
        }
        // reduce over lane bit 5 (and 4) with permlane swaps: each lane keeps
        // half (a quarter) of the columns, summed over the swapped lanes
        float q[8];
#pragma unroll
        for (int k = 0; k < 8; k++) {
            auto s2 = __builtin_amdgcn_permlane32_swap((unsigned)f2i(p[2 * k]),
                                                       (unsigned)f2i(p[2 * k + 1]), false, false);
            q[k] = i2f((int)s2[0]) + i2f((int)s2[1]);
        }
        const int b5 = (lane >> 5) & 1;
        const int b4 = (lane >> 4) & 1;
        const int sub = (NSUB == 2) ? ((lane >> 2) & 1) : 0;
        float* part = colpart + (wave * NSUB + sub) * D + ch0;
        if constexpr (NPART == 4) {
#pragma unroll
            for (int k = 0; k < 4; k++) {
                auto s2 = __builtin_amdgcn_permlane16_swap((unsigned)f2i(q[2 * k]),
                                                           (unsigned)f2i(q[2 * k + 1]), false, false);
                part[4 * k + 2 * b4 + b5] = i2f((int)s2[0]) + i2f((int)s2[1]);
            }
        } else {
#pragma unroll
            for (int k = 0; k < 8; k++) part[2 * k + b5] = q[k];
        }
        __syncthreads();
        if (tid < D) {
            float s = 0.f;
#pragma unroll
            for (int w = 0; w < NW * NSUB; w++) s += colpart[w * D + tid];
            float b = bvec[tid];
            if (usable(s)) b = (float)T * __builtin_amdgcn_rcpf(s);
            bvec[tid] = b;
            if (last) {
                // channel sign left by the sign-tracked butterflies: (-1)^popcount(j >> 4)
                const float sg = (!MfmaRotation<D>::on && (__builtin_popcount((unsigned)tid >> 4) & 1)) ? -1.f : 1.f;
                icvec[tid] = sg * sqrtf(b);
                cvec[tid] = (uint16_t)float_to_half_bits(__builtin_amdgcn_rsqf((float)D * b));
            }
        }
        __syncthreads();
        if (last) break;
#pragma unroll
        for (int c4 = 0; c4 < QC / 4; c4++) {
            float4 v = *reinterpret_cast<const float4*>(bvec + ch0 + 4 * c4);
            bw[4 * c4 + 0] = v.x;
            bw[4 * c4 + 1] = v.y;
            bw[4 * c4 + 2] = v.z;
            bw[4 * c4 + 3] = v.w;
        }
        // row step
#pragma unroll
        for (int r = 0; r < QR; r++) {
            float s = A[r][0] * bw[0];
#pragma unroll
            for (int c = 1; c < QC; c++) s = fmaf(A[r][c], bw[c], s);
            s = row_sum<CGB>(s);
            if (usable(s)) aw[r] = (float)D * __builtin_amdgcn_rcpf(s);
        }
    }

    // ---- stage 4: per-token asymmetric round-to-nearest, packed in LDS ------
    float ic[QC];
#pragma unroll
    for (int c4 = 0; c4 < QC / 4; c4++) {
        float4 v = *reinterpret_cast<const float4*>(icvec + ch0 + 4 * c4);
        ic[4 * c4 + 0] = v.x;
        ic[4 * c4 + 1] = v.y;
        ic[4 * c4 + 2] = v.z;
        ic[4 * c4 + 3] = v.w;
    }
    uint8_t* img = smem;  // image of the record's code block
    uint32_t sz[QR];
    uint32_t fq[QR][QC];  // magic-rounded codes
#pragma unroll
    for (int r = 0; r < QR; r++) {
        float W[QC];
#pragma unroll
        for (int c = 0; c < QC; c++) {
            float yv;
            if constexpr (KEEP_Y) {
                yv = y[r][c];
            } else {
                yv = sqrtf(A[r][c]);
                if ((negbits[r] >> c) & 1u) yv = -yv;
            }
            W[c] = yv * ic[c];
        }
        float mn = W[0], mx = W[0];
#pragma unroll
        for (int c = 1; c < QC; c++) {
            mn = fminf(mn, W[c]);
            mx = fmaxf(mx, W[c]);
        }
        row_minmax<CGB>(mn, mx);
        mn += 0.0f;  // a zero row stores +0, not the -0 of a sign-flipped channel
        const float range = mx - mn;
        const float s = range * (1.0f / (float)QMAX);
        const float inv = range > 0.f ? (float)QMAX * __builtin_amdgcn_rcpf(range) : 0.f;
        const float nb = -mn * inv;
        sz[r] = float_to_half_bits(s) | (float_to_half_bits(mn) << 16);
#pragma unroll
        for (int c = 0; c < QC; c++) fq[r][c] = fbits(fmaf(W[c], inv, nb) + kMagic);
    }
    // the statistics are done with the shared buffer (last barrier above);
    // the record's code image reuses it
    if constexpr (!CHMAJOR) {
        // token-major: this lane's 16 codes of a row are contiguous
#pragma unroll
        for (int r = 0; r < QR; r++) {
            const uint32_t* f = fq[r];
            uint8_t* dstp = img + ((row0 + r) * D + ch0) * BITS / 8;
            if constexpr (BITS == 4) {
                uint32_t pr[8];
#pragma unroll
                for (int k = 0; k < 8; k++) pr[k] = pack2<4>(f[2 * k], f[2 * k + 1]);
                uint2 v = make_uint2(bytes4(pr[0], pr[1], pr[2], pr[3]), bytes4(pr[4], pr[5], pr[6], pr[7]));
                *reinterpret_cast<uint2*>(dstp) = v;
            } else if constexpr (BITS == 2) {
                uint32_t qd[4];
#pragma unroll
                for (int k = 0; k < 4; k++)
                    qd[k] = (pack2<2>(f[4 * k + 2], f[4 * k + 3]) << 4) + pack2<2>(f[4 * k], f[4 * k + 1]);
                *reinterpret_cast<uint32_t*>(dstp) = bytes4(qd[0], qd[1], qd[2], qd[3]);
            } else {
                uint32_t g[4];
#pragma unroll
                for (int k = 0; k < 4; k++) g[k] = pack6x4(f[4 * k], f[4 * k + 1], f[4 * k + 2], f[4 * k + 3]);
                uint32_t* d32 = reinterpret_cast<uint32_t*>(dstp);
                d32[0] = g[0] | (g[1] << 24);
                d32[1] = (g[1] >> 8) | (g[2] << 16);
                d32[2] = (g[2] >> 16) | (g[3] << 8);
            }
        }
    } else {
        // channel-major: this lane's 4 tokens of a channel are contiguous
#pragma unroll
        for (int c = 0; c < QC; c++) {
            const int e0 = (ch0 + c) * T + row0;  // element index of the first of 4 codes
            if constexpr (BITS == 2) {
                const uint32_t v = (pack2<2>(fq[2][c], fq[3][c]) << 4) + pack2<2>(fq[0][c], fq[1][c]);
                img[e0 / 4] = (uint8_t)v;
            } else if constexpr (BITS == 4) {
                const uint32_t v = __builtin_amdgcn_perm(pack2<4>(fq[2][c], fq[3][c]),
                                                         pack2<4>(fq[0][c], fq[1][c]), 0x0c0c0400u);
                *reinterpret_cast<uint16_t*>(img + e0 / 2) = (uint16_t)v;
            } else {
                const uint32_t v = pack6x4(fq[0][c], fq[1][c], fq[2][c], fq[3][c]);
                uint8_t* d8 = img + e0 * 6 / 8;
                d8[0] = (uint8_t)v;
                d8[1] = (uint8_t)(v >> 8);
                d8[2] = (uint8_t)(v >> 16);
            }
        }
    }
    // per-token scale and zero-point: 4 consecutive tokens = 16 bytes
    if (cg == 0) {
        *reinterpret_cast<uint4*>(rec + CODE_BYTES + 4 * row0) = make_uint4(sz[0], sz[1], sz[2], sz[3]);
    }
    // column scales, normalized basis
    if (tid < D / 8) {
        *reinterpret_cast<uint4*>(rec + CODE_BYTES + 4 * T + 16 * tid) =
            *reinterpret_cast<const uint4*>(cvec + 8 * tid);
    }
    __syncthreads();

    // ---- stage 5: the code image leaves in 16-byte stores -------------------
    {
        constexpr int PER = CODE_BYTES / NT;   // 8 * BITS bytes per thread
        const uint4* src4 = reinterpret_cast<const uint4*>(img + tid * PER);
        uint4* dst4 = reinterpret_cast<uint4*>(rec + (int64_t)tid * PER);
#pragma unroll
        for (int k = 0; k < PER / 16; k++) dst4[k] = src4[k];
    }
}

// One launch quantizes keys and values (or the MLA latent): workgroup
// 2*(i*H + h) + kind takes page i, head h, kind 0 = keys (token-major codes),
// kind 1 = values (channel-major codes).
template <int D, int T, int KB, int VB, bool HASV>
__global__ void __launch_bounds__(T * D / 64)
quantize_kernel(const uint16_t* __restrict__ kpool, const uint16_t* __restrict__ vpool,
                uint8_t* __restrict__ krec, uint8_t* __restrict__ vrec, const int32_t* __restrict__ src,
                const int32_t* __restrict__ dst, int32_t H, int64_t n_fpages, int64_t n_qpages, int32_t n_iters) {
    using S = TileShape<D, T>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[S::SMEM];
    __shared__ __attribute__((aligned(16))) float vec[3 * D];
    const int kind = HASV ? (int)(blockIdx.x & 1u) : 0;
    const int r = HASV ? (int)(blockIdx.x >> 1) : (int)blockIdx.x;
    const int i = r / H;
    const int h = r - i * H;
    const int sp = src[i];
    const int dp = dst[i];
    if (sp < 0 || (int64_t)sp >= n_fpages || dp < 0 || (int64_t)dp >= n_qpages) return;
    const int64_t tile_off = ((int64_t)sp * H + h) * (int64_t)(T * D);
    if (kind == 0) {
        constexpr int REC = T * D * KB / 8 + 4 * T + 2 * D;
        quantize_tile<D, T, KB, false>(kpool + tile_off, krec + ((int64_t)dp * H + h) * REC, smem, vec, n_iters);
    } else if constexpr (HASV) {
        constexpr int REC = T * D * VB / 8 + 4 * T + 2 * D;
        quantize_tile<D, T, VB, true>(vpool + tile_off, vrec + ((int64_t)dp * H + h) * REC, smem, vec, n_iters);
    }
}

}  // namespace

template <int D, int T, int KB, int VB, bool HASV>
hipError_t launch_quantize_shape(const QuantizeArgs& a, hipStream_t st) {
    const int64_t blocks = (int64_t)a.n * a.H * (HASV ? 2 : 1);
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((quantize_kernel<D, T, KB, VB, HASV>), dim3((unsigned)blocks), dim3(T * D / 64), 0, st,
                       static_cast<const uint16_t*>(a.k_fp16), static_cast<const uint16_t*>(a.v_fp16),
                       static_cast<uint8_t*>(a.k_records), static_cast<uint8_t*>(a.v_records), a.src, a.dst, a.H,
                       a.n_fpages, a.n_qpages, a.n_iters);
    return hipGetLastError();
}

#define KVARN_QUANTIZE_INSTANTIATE_D(D)                                                        \
    template hipError_t launch_quantize_shape<D, 128, 2, 2, true>(const QuantizeArgs&, hipStream_t); \
    template hipError_t launch_quantize_shape<D, 128, 2, 4, true>(const QuantizeArgs&, hipStream_t); \
    template hipError_t launch_quantize_shape<D, 128, 2, 6, true>(const QuantizeArgs&, hipStream_t); \
    template hipError_t launch_quantize_shape<D, 128, 4, 2, true>(const QuantizeArgs&, hipStream_t); \
    template hipError_t launch_quantize_shape<D, 128, 4, 4, true>(const QuantizeArgs&, hipStream_t); \
    template hipError_t launch_quantize_shape<D, 128, 4, 6, true>(const QuantizeArgs&, hipStream_t); \
    template hipError_t launch_quantize_shape<D, 128, 6, 2, true>(const QuantizeArgs&, hipStream_t); \
    template hipError_t launch_quantize_shape<D, 128, 6, 4, true>(const QuantizeArgs&, hipStream_t); \
    template hipError_t launch_quantize_shape<D, 128, 6, 6, true>(const QuantizeArgs&, hipStream_t); \
    template hipError_t launch_quantize_shape<D, 64, 2, 2, true>(const QuantizeArgs&, hipStream_t);  \
    template hipError_t launch_quantize_shape<D, 64, 2, 4, true>(const QuantizeArgs&, hipStream_t);  \
    template hipError_t launch_quantize_shape<D, 64, 2, 6, true>(const QuantizeArgs&, hipStream_t);  \
    template hipError_t launch_quantize_shape<D, 64, 4, 2, true>(const QuantizeArgs&, hipStream_t);  \
    template hipError_t launch_quantize_shape<D, 64, 4, 4, true>(const QuantizeArgs&, hipStream_t);  \
    template hipError_t launch_quantize_shape<D, 64, 4, 6, true>(const QuantizeArgs&, hipStream_t);  \
    template hipError_t launch_quantize_shape<D, 64, 6, 2, true>(const QuantizeArgs&, hipStream_t);  \
    template hipError_t launch_quantize_shape<D, 64, 6, 4, true>(const QuantizeArgs&, hipStream_t);  \
    template hipError_t launch_quantize_shape<D, 64, 6, 6, true>(const QuantizeArgs&, hipStream_t);

}  // namespace kvarn
