// KVarN quantize kernel for gfx950 (templates; instantiated per head_dim in
// quantize_d128.hip, quantize_d256.hip and quantize_d512.hip).
//
// One workgroup turns one fp16 tile (T tokens x D channels of one KV head)
// into one record: Hadamard rotation across channels, column/row
// normalization iterations, per-token asymmetric round-to-nearest, packed
// codes (evermx.com KVarN review, method paragraph: the four stages; gmlx
// "KV cache quantization", "The two schemes": per-head Hadamard rotation,
// records whose token and channel spreads are evened out).
//
// Register layout: every lane holds R = 4 consecutive tokens x C = 16
// consecutive channels (64 values).  D/16 lanes share a token row; their
// lane-index bits carry the channel group and are chosen among bits 0, 1, 3
// (DPP patterns: quad_perm and row_ror:8), then 2 and 4 (ds_swizzle).  The
// remaining lane bits (of 2, 4, 5) and the wave index carry the row group.
//
// The rotation is the unnormalized +-1 Hadamard product: on the fp16 MFMA
// for D = 128 and 256; for D = 512 as butterflies (4 in-lane stages, then
// one cross-lane stage per channel-group bit).  Statistics use the squared tile
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

// Row k = 2 b0 + b1 of this lane's quad (b0, b1: lane bits 0 and 1) from
// the per-lane values v[0..3] of the lane's 4 rows: the value of row k sits
// in quad lane b0 + 2 b1, so rows 0..3 come from quad lanes 0, 2, 1, 3.
__device__ __forceinline__ void quad_bcast_rows(float v, float (&out)[4]) {
    out[0] = i2f(__builtin_amdgcn_mov_dpp(f2i(v), 0x00, 0xF, 0xF, false));
    out[1] = i2f(__builtin_amdgcn_mov_dpp(f2i(v), 0xAA, 0xF, 0xF, false));
    out[2] = i2f(__builtin_amdgcn_mov_dpp(f2i(v), 0x55, 0xF, 0xF, false));
    out[3] = i2f(__builtin_amdgcn_mov_dpp(f2i(v), 0xFF, 0xF, 0xF, false));
}

// Minimum and maximum over the D/16 lanes of a token row, reduce-scattered:
// over lane bits 0 and 1 each lane keeps one of its quad's rows (row
// 2 b0 + b1) and passes the other on, then the remaining channel-group bits
// combine that row (bit 3 by DPP, bits 2 and 4 by ds_swizzle).
template <int CGB>
__device__ __forceinline__ void row_minmax_scatter(const float (&mn)[4], const float (&mx)[4], bool b0, bool b1,
                                                   float& mnk, float& mxk) {
    auto x1 = [](float v) { return i2f(__builtin_amdgcn_update_dpp(0, f2i(v), 0xB1, 0xF, 0xF, true)); };
    auto x2 = [](float v) { return i2f(__builtin_amdgcn_update_dpp(0, f2i(v), 0x4E, 0xF, 0xF, true)); };
    auto x8 = [](float v) { return i2f(__builtin_amdgcn_update_dpp(0, f2i(v), 0x128, 0xF, 0xF, true)); };
    const float n02 = fminf(b0 ? mn[2] : mn[0], x1(b0 ? mn[0] : mn[2]));
    const float n13 = fminf(b0 ? mn[3] : mn[1], x1(b0 ? mn[1] : mn[3]));
    const float m02 = fmaxf(b0 ? mx[2] : mx[0], x1(b0 ? mx[0] : mx[2]));
    const float m13 = fmaxf(b0 ? mx[3] : mx[1], x1(b0 ? mx[1] : mx[3]));
    float n = fminf(b1 ? n13 : n02, x2(b1 ? n02 : n13));
    float m = fmaxf(b1 ? m13 : m02, x2(b1 ? m02 : m13));
    n = fminf(n, x8(n));
    m = fmaxf(m, x8(m));
    if constexpr (CGB >= 4) { n = fminf(n, xor_lane<2>(n)); m = fmaxf(m, xor_lane<2>(m)); }
    if constexpr (CGB >= 5) { n = fminf(n, xor_lane<4>(n)); m = fmaxf(m, xor_lane<4>(m)); }
    mnk = n;
    mxk = m;
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
        // ds_swizzle stages: keep at most one row's 16 exchanges in flight
        // (hoisting all 64 would need 64 more registers)
        if constexpr (BIT == 2 || BIT == 4) __builtin_amdgcn_sched_barrier(0);
    }
}

// |a| * b + c in one v_fma_f32 with the abs source modifier.  Written as an
// instruction so that |a| is never materialized (the compiler would hoist
// it out of the iteration loop and hold both a and |a| in registers).
__device__ __forceinline__ float fma_abs(float a, float b, float c) {
    float d;
    asm("v_fma_f32 %0, |%1|, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
    return d;
}
__device__ __forceinline__ float mul_abs(float a, float b) {
    float d;
    asm("v_mul_f32_e64 %0, |%1|, %2" : "=v"(d) : "v"(a), "v"(b));
    return d;
}

// finite and > 0: positive denormal or normal (one v_cmp_class)
__device__ __forceinline__ bool usable(float s) { return __builtin_amdgcn_classf(s, 0x180); }

__device__ __forceinline__ uint32_t fbits(float x) { return __builtin_bit_cast(uint32_t, x); }

// 6-bit codes sit in the low bits of magic-rounded floats (junk from bit 22 up).
// 4 codes of 6 bits -> low 24 bits (clean above).
__device__ __forceinline__ uint32_t pack6x4(uint32_t f0, uint32_t f1, uint32_t f2, uint32_t f3) {
    const uint32_t x01 = ((f1 << 6) + f0) & 0xfffu;
    const uint32_t x23 = (f3 << 6) + f2;   // bits 12..27 zero, junk from 28
    return (x23 << 12) | x01;              // junk shifted out
}

// D = 128, 256: the rotation runs on the 16x16x32 fp16 MFMA (y = X H with
// the fp16 tile as the A operand and +-1 blocks of H as the B operand) and
// reaches the register layout through LDS; D = 128 with each wave on its own
// 32 rows, D = 256 on its own 16 rows.  D = 512 (one 16-wave workgroup per
// CU, 8 rows per wave) keeps the butterflies: the MFMA form needs two waves
// per 16-row block and workgroup barriers, which measured slower there.  The
// sign-tracked cross-lane butterflies leave channel j multiplied by
// (-1)^popcount(j >> 4), undone with the column scales.
template <int D>
struct MfmaRotation {
    static constexpr bool narrow = D == 128;
    static constexpr bool wide = D == 256;
    static constexpr unsigned XMASK = (narrow || wide) ? 0u : (unsigned)(D / 16 - 1);  // bits of j >> 4
};

// B operands of the rotation.  H_128 = H_4 (x) H_32 over channel j = 32 v + u
// (popcount of (32 v + u) & (32 v' + u') splits over the two factors).  Lane
// l of a 16x16x32 B operand holds rows k = 8 (l >> 4) + i, i = 0..7, of
// column n = l & 15; with k = u and n = u' - 16 nb that is
// H_32[u][u'] = (-1)^(popcount(i & n & 7) + ((l >> 4) & 1) (n >> 3) + (l >> 5) nb).
// Entry [nb + 2 s][l] is lane l's operand for column block nb times (-1)^s,
// the H_4 sign of an input group / output group pair; 8 fp16 +-1 per lane.
struct RotOperands {
    uint32_t w[4][64][4];
};
constexpr RotOperands make_rot_operands() {
    RotOperands t{};
    for (int sn = 0; sn < 4; sn++) {
        const int nb = sn & 1, neg = sn >> 1;
        for (int l = 0; l < 64; l++) {
            const int n = l & 15, g4 = l >> 4;
            for (int k = 0; k < 4; k++) {
                uint32_t d = 0x3C003C00u;
                for (int half = 0; half < 2; half++) {
                    const int i = 2 * k + half;
                    const int par = __builtin_popcount((unsigned)(i & n & 7)) + ((g4 & 1) & (n >> 3)) + ((g4 >> 1) & nb) + neg;
                    if (par & 1) d |= 0x8000u << (16 * half);
                }
                t.w[sn][l][k] = d;
            }
        }
    }
    return t;
}
__device__ const RotOperands kRotOperands = make_rot_operands();

// B operands of the wide rotation: column n of half nh is channel
// 16 (n >> 3) + 8 nh + (n & 7) of the 32-channel group, so that an output
// block holds channels 8 nh .. 8 nh + 7 of two 16-channel blocks.  Entry
// [nh + 2 s][l] is lane l's operand times (-1)^s.
constexpr RotOperands make_rot_operands_split() {
    RotOperands t{};
    for (int sn = 0; sn < 4; sn++) {
        const int nh = sn & 1, neg = sn >> 1;
        for (int l = 0; l < 64; l++) {
            const int n = l & 15, col = 16 * (n >> 3) + 8 * nh + (n & 7);
            for (int k = 0; k < 4; k++) {
                uint32_t d = 0x3C003C00u;
                for (int half = 0; half < 2; half++) {
                    const int row = 8 * (l >> 4) + 2 * k + half;
                    if ((__builtin_popcount((unsigned)(row & col)) + neg) & 1) d |= 0x8000u << (16 * half);
                }
                t.w[sn][l][k] = d;
            }
        }
    }
    return t;
}
__device__ const RotOperands kRotOperandsSplit = make_rot_operands_split();

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
    // rotation image: D = 128 half the rotated tile (fp32); D = 256 half of
    // each wave's 16 x 256 block (fp32), 8 KB per wave
    static constexpr int SMEM_ROT = MfmaRotation<D>::narrow ? T * D * 2 : MfmaRotation<D>::wide ? NW * 8192 : 0;
    static constexpr int SMEM_A = SMEM_CODES > SMEM_PART ? SMEM_CODES : SMEM_PART;
    // D = 128: the column partials get their own region after the rotation
    // image, so the statistics need not wait for every wave's image to die;
    // D = 256 ends the rotation with a workgroup barrier and reuses it
    static constexpr int PART_OFF = MfmaRotation<D>::narrow ? (SMEM_ROT > SMEM_CODES ? SMEM_ROT : SMEM_CODES) : 0;
    static constexpr int SMEM = MfmaRotation<D>::narrow ? PART_OFF + SMEM_PART : (SMEM_A > SMEM_ROT ? SMEM_A : SMEM_ROT);
};

// LDS position of channel ch in a slot of column partials: 4-float chunks xor-permuted inside each 8-chunk (32-float) window
// with tau = bit 5 of ch | (bit 7 of ch ^ slot) << 1.  The lanes of any
// 8-lane group (which differ in channel-group bits 0, 1 and 3, or 0 and 1
// and the partial slot for D = 128) then touch 8 different 4-bank groups.
__device__ __forceinline__ int chan_pos(int ch, int slot) {
    const int tau = ((ch >> 5) & 1) | ((((ch >> 7) ^ slot) & 1) << 1);
    return (((ch >> 2) ^ tau) << 2) | (ch & 3);
}

// D = 128: y = X H for this lane's 4 rows x 16 channels (MFMA, then LDS;
// the wave's own 8 KB of smem).
template <int D, int T>
__device__ __forceinline__ void mfma_rotate(const uint16_t* __restrict__ tile, uint8_t* smem, int lane, int wave,
                                            int cg, int rg, float (&y)[QR][QC]) {
    using S = TileShape<D, T>;
    constexpr int RGB = S::RGB, CGB = S::CGB, RPW = S::RPW;
    // ---- stages 1-2: y = X H on the MFMA, then into the register layout ----
    // Output group v' (channels 32 v' .. 32 v' + 31) of a 16-row block is
    // sum_v X_v H_32 (-1)^popcount(v & v'): four chained MFMAs, the H_4
    // sign carried by the B operand.
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    typedef float f4 __attribute__((ext_vector_type(4)));
    static_assert(RGB == 3 && CGB == 3 && RPW == 32, "rotation layout assumes 32 rows x 128 channels per wave");
    const int l16 = lane & 15, g4 = lane >> 4;
    h8 hb[4];
#pragma unroll
    for (int sn = 0; sn < 4; sn++)
        hb[sn] = __builtin_bit_cast(h8, *reinterpret_cast<const uint4*>(kRotOperands.w[sn][lane]));
    f4 z[2][4][2];  // [token block][output group v'][nb]
#pragma unroll
    for (int tb = 0; tb < 2; tb++) {
        const uint16_t* xr = tile + (int64_t)(wave * RPW + 16 * tb + l16) * D + 8 * g4;
        h8 xa[4];
#pragma unroll
        for (int v = 0; v < 4; v++) xa[v] = *reinterpret_cast<const h8*>(xr + 32 * v);
#pragma unroll
        for (int v = 0; v < 4; v++)
#pragma unroll
            for (int vo = 0; vo < 4; vo++)
#pragma unroll
                for (int nb = 0; nb < 2; nb++) {
                    const int sn = nb + 2 * (__builtin_popcount((unsigned)(v & vo)) & 1);
                    z[tb][vo][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        xa[v], hb[sn], v == 0 ? f4{0.f, 0.f, 0.f, 0.f} : z[tb][vo][nb], 0, 0, 0);
                }
    }
    // Through LDS, 64 columns at a time.  Column j (of the half), rows
    // 4 ru .. 4 ru + 3 of the wave's 32 rows sit in the 16-byte unit
    // 8 j + (ru ^ ((j ^ (j >> 3)) & 7)): the MFMA-layout stores and the
    // register-layout loads each touch every bank once.  For the stores
    // (j = 32 vq + 16 nb + l16, ru = 4 tb + g4) and the loads
    // (j = 16 (cg & 3) + c, ru = rg) the unit splits into a per-lane part
    // and a compile-time xor and offset.
    const uint32_t wbase = (uint32_t)wave * (uint32_t)(RPW * D / 2 * 4);
    const uint32_t wa = wbase + 128u * (uint32_t)l16 + 16u * (uint32_t)(g4 ^ (l16 & 7) ^ (l16 >> 3));
    const uint32_t cq = (uint32_t)(lane & 3);  // cg & 3
    const uint32_t ra = wbase + 2048u * cq + 16u * ((uint32_t)rg ^ (2u * cq));
#pragma unroll
    for (int half = 0; half < 2; half++) {
        // output columns 32 v + 16 nb + l16 with v = 2 half + vq
#pragma unroll
        for (int tb = 0; tb < 2; tb++)
#pragma unroll
            for (int vq = 0; vq < 2; vq++)
#pragma unroll
                for (int nb = 0; nb < 2; nb++)
                    *reinterpret_cast<f4*>(smem + ((wa ^ (uint32_t)(64 * (tb ^ vq) + 32 * nb)) + 4096u * vq + 2048u * nb)) =
                        z[tb][2 * half + vq][nb];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if ((cg >> 2) == half) {
#pragma unroll
            for (int c = 0; c < QC; c++) {
                const f4 v = *reinterpret_cast<const f4*>(smem + ((ra ^ (uint32_t)(16 * ((c & 7) ^ (c >> 3)))) + 128u * c));
#pragma unroll
                for (int r = 0; r < QR; r++) y[r][c] = v[r];
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

// D = 256: y = X H_256 for this lane's 4 rows x 16 channels (MFMA, then
// LDS; the wave's own 8 KB of smem).  H_256 = H_8 (x) H_32: output group og
// (32 channels) of the wave's 16 rows is sum_j X_j H_32 (-1)^popcount(j & og),
// eight chained MFMAs per 16-column half.  Pass p moves channels 8 p ..
// 8 p + 7 of every 16-channel block (the output blocks of B-operand half p)
// through 16-byte units [row quad][16-channel block cb][c ^ ((cb >> 1) & 7)],
// c = channel - 16 cb - 8 p: the MFMA-layout stores and the register-layout
// loads of 16 lanes touch 16 different units modulo 16, and every lane loads
// in both passes.
template <int D, int T>
__device__ __forceinline__ void mfma_rotate_wide(const uint16_t* __restrict__ tile, uint8_t* smem, int lane, int wave,
                                                 int cg, int rg, float (&y)[QR][QC]) {
    using S = TileShape<D, T>;
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    typedef float f4 __attribute__((ext_vector_type(4)));
    static_assert(D == 256 && S::RPW == 16 && S::RGB == 2, "one wave per 16 rows x 256 channels");
    constexpr int NCB = D / 16;           // 16-channel blocks
    const int l16 = lane & 15, g4 = lane >> 4;
    uint8_t* region = smem + wave * 8192;
    h8 hb[4];
#pragma unroll
    for (int sn = 0; sn < 4; sn++)
        hb[sn] = __builtin_bit_cast(h8, *reinterpret_cast<const uint4*>(kRotOperandsSplit.w[sn][lane]));
    // A operands: row 16 wave + l16, input group j, channels 32 j + 8 g4 .. + 7
    h8 xa[8];
    {
        const uint16_t* xr = tile + (int64_t)(16 * wave + l16) * D + 8 * g4;
#pragma unroll
        for (int j = 0; j < 8; j++) xa[j] = *reinterpret_cast<const h8*>(xr + 32 * j);
    }
    auto unit = [](int qq, int cb, int c) { return 16 * (qq * 8 * NCB + 8 * cb + (c ^ ((cb >> 1) & 7))); };
    auto block = [&](int p, int og) -> f4 {
        f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const int sn = p + 2 * (__builtin_popcount((unsigned)(j & og)) & 1);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[j], hb[sn], acc, 0, 0, 0);
        }
        return acc;
    };
    // output block (p, og): channel 32 og + 16 (l16 >> 3) + 8 p + (l16 & 7), rows 4 g4 .. 4 g4 + 3
    auto store = [&](int og, f4 zv) {
        *reinterpret_cast<f4*>(region + unit(g4, 2 * og + (l16 >> 3), l16 & 7)) = zv;
    };
    // this lane: rows 4 rg .. 4 rg + 3 (rg = g4), channels 16 cg + 8 p + c
    auto load = [&](int p) {
#pragma unroll
        for (int c = 0; c < 8; c++) {
            const f4 v = *reinterpret_cast<const f4*>(region + unit(rg, cg, c));
#pragma unroll
            for (int r = 0; r < QR; r++) y[r][8 * p + c] = v[r];
        }
    };
    auto sync = []() {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
    // pass 0's blocks go to LDS as they are formed, pass 1's wait in
    // registers until pass 0 has been read back: y is born only after the
    // MFMA operands have died
#pragma unroll
    for (int og = 0; og < 8; og++) store(og, block(0, og));
    __builtin_amdgcn_sched_barrier(0);
    f4 z1[8];
#pragma unroll
    for (int og = 0; og < 8; og++) z1[og] = block(1, og);
    sync();
    load(0);
    sync();
#pragma unroll
    for (int og = 0; og < 8; og++) store(og, z1[og]);
    sync();
    load(1);
    // the statistics reuse the shared buffer
    __syncthreads();
}

// Position of channel ch in the b and sqrt(b) vectors: 4 pad floats after
// every 32 channels, so that the 16-byte broadcast reads of channel groups
// 16 cg .. 16 cg + 15 (cg = 0..3 within an 8-lane group) start in different
// bank quads.
__device__ __forceinline__ constexpr int vec_pos(int ch) { return ch + 4 * (ch >> 5); }
template <int D>
struct VecShape {
    static constexpr int PADDED = D + D / 8;       // floats per padded vector
    static constexpr int FLOATS = 2 * PADDED + D / 2;  // b, sqrt b, fp16 column scales
};

// One tile -> one record.  smem: TileShape::SMEM bytes; vec: VecShape::FLOATS floats.
template <int D, int T, int BITS, bool CHMAJOR>
__device__ __forceinline__ void quantize_tile(const uint16_t* __restrict__ tile, uint8_t* __restrict__ rec,
                                              uint8_t* smem, float* vec, int32_t n_iters) {
    using S = TileShape<D, T>;
    constexpr int CGB = S::CGB, RGB = S::RGB, RPW = S::RPW, NW = S::NW, NT = S::NT, NSUB = S::NSUB;
    constexpr int QMAX = (1 << BITS) - 1;
    constexpr int CODE_BYTES = T * D * BITS / 8;
    constexpr int REC = CODE_BYTES + 4 * T + 2 * D;
    constexpr int NPART = (RGB >= 2) ? 4 : 8;          // column partials per lane after swaps
    constexpr bool KEEP_Y = D <= 128;                  // D = 256, 512 keep y |y| and rebuild y from it
    static_assert(T * D / 64 == NT, "one lane per 64 values");
    static_assert(REC % 16 == 0, "records stay 16-byte aligned");
    // widths 2, 4, 6 pack in registers; 3, 5 and 8 go through an image of one
    // byte per code (record order), which for 8 bits is the record itself
    constexpr bool BYTE_IMAGE = BITS == 3 || BITS == 5 || BITS == 8;
    static_assert(BITS == 2 || BITS == 3 || BITS == 4 || BITS == 5 || BITS == 6 || BITS == 8, "code width");
    // channel-major codes go in blocks of TB tokens (record format: block by
    // block, each channel's TB codes in a row), so a 64-token step of the
    // decode reads one contiguous run
    constexpr int TB = T < 64 ? T : 64;
    static_assert(T % TB == 0 && TB % 4 == 0, "whole token blocks; a lane's 4 tokens in one block");
    static_assert(BYTE_IMAGE || CODE_BYTES + (T / TB) * 4 * (D / 16) <= S::SMEM_CODES,
                  "the code image and its channel-row pads fit");
    static_assert(T * D <= S::SMEM_CODES, "one byte per code fits");

    float* colpart = reinterpret_cast<float*>(smem + S::PART_OFF);
    float* bvec = vec;           // b_j = exp(-2 lc_j), unnormalized basis
    float* icvec = vec + VecShape<D>::PADDED;  // (+-1 per channel) * sqrt(b_j): multiplies y into W
    uint16_t* cvec = reinterpret_cast<uint16_t*>(vec + 2 * VecShape<D>::PADDED);  // fp16 column scales

    const int tid = tid_x();
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

    if (tid < D) bvec[vec_pos(tid)] = 1.0f / (float)D;  // c_j = 1 in the normalized basis
    float y[QR][QC];
    if constexpr (MfmaRotation<D>::narrow) {
        mfma_rotate<D, T>(tile, smem, lane, wave, cg, rg, y);
    } else if constexpr (MfmaRotation<D>::wide) {
        mfma_rotate_wide<D, T>(tile, smem, lane, wave, cg, rg, y);
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
    // A holds y^2 (D = 512: y |y|, the sign of y on y^2; the statistics read
    // |A| through the free abs source modifier)
    float A[QR][QC];
#pragma unroll
    for (int r = 0; r < QR; r++)
#pragma unroll
        for (int c = 0; c < QC; c++) A[r][c] = KEEP_Y ? y[r][c] * y[r][c] : y[r][c] * fabsf(y[r][c]);

    // Row weights are kept as a / D (exact: D is a power of two), so the row
    // step is a bare reciprocal; the column step's T / D restores b.
    constexpr float kInvD = 1.0f / (float)D;
    float aw[QR] = {kInvD, kInvD, kInvD, kInvD};
    float my_a = kInvD;  // a / D of this lane's row in the row step's reduce-scatter
    const bool rb0 = lane & 1, rb1 = (lane >> 1) & 1;
    float bw[QC];
    for (int it = 0; it < n_iters; it++) {
        const bool last = it == n_iters - 1;
        // column step: partial sums over this lane's rows
        float p[QC];
#pragma unroll
        for (int c = 0; c < QC; c++) {
            float s;
            if constexpr (KEEP_Y) {
                s = A[0][c] * aw[0];
#pragma unroll
                for (int r = 1; r < QR; r++) s = fmaf(A[r][c], aw[r], s);
            } else {
                s = mul_abs(A[0][c], aw[0]);
#pragma unroll
                for (int r = 1; r < QR; r++) s = fma_abs(A[r][c], aw[r], s);
            }
            p[c] = s;
        }
        // reduce over lane bit 5 (and 4) with permlane swaps: the lower half
        // keeps the first argument's column, the upper half the second's, so
        // a lane ends with channels ch0 + 8 b5 (+ 4 b4) + 0..NPART-1, stored
        // as 4-float chunks
        float q[8];
#pragma unroll
        for (int k = 0; k < 8; k++) {
            auto s2 = __builtin_amdgcn_permlane32_swap((unsigned)f2i(p[k]), (unsigned)f2i(p[k + 8]), false, false);
            q[k] = i2f((int)s2[0]) + i2f((int)s2[1]);
        }
        const int b5 = (lane >> 5) & 1;
        const int b4 = (lane >> 4) & 1;
        const int sub = (NSUB == 2) ? ((lane >> 2) & 1) : 0;
        const int slot = wave * NSUB + sub;
        float* part = colpart + slot * D;
        if constexpr (NPART == 4) {
            float4 v;
            float* vv = reinterpret_cast<float*>(&v);
#pragma unroll
            for (int k = 0; k < 4; k++) {
                auto s2 = __builtin_amdgcn_permlane16_swap((unsigned)f2i(q[k]), (unsigned)f2i(q[k + 4]), false, false);
                vv[k] = i2f((int)s2[0]) + i2f((int)s2[1]);
            }
            *reinterpret_cast<float4*>(part + chan_pos(ch0 + 8 * b5 + 4 * b4, slot)) = v;
        } else {
#pragma unroll
            for (int h = 0; h < 2; h++)
                *reinterpret_cast<float4*>(part + chan_pos(ch0 + 8 * b5 + 4 * h, slot)) =
                    make_float4(q[4 * h], q[4 * h + 1], q[4 * h + 2], q[4 * h + 3]);
        }
        __syncthreads();
        if (tid < D) {
            float s = 0.f;
#pragma unroll
            for (int w = 0; w < NW * NSUB; w++) s += colpart[w * D + chan_pos(tid, w)];
            const int pt = vec_pos(tid);
            float b = bvec[pt];
            if (usable(s)) b = ((float)T / (float)D) * __builtin_amdgcn_rcpf(s);
            bvec[pt] = b;
            if (last) {
                // channel sign left by the sign-tracked cross-lane butterflies
                const float sg = (__builtin_popcount(((unsigned)tid >> 4) & MfmaRotation<D>::XMASK) & 1)
                                     ? -1.f : 1.f;
                icvec[pt] = sg * sqrtf(b);
                cvec[tid] = (uint16_t)float_to_half_bits(__builtin_amdgcn_rsqf((float)D * b));
            }
        }
        __syncthreads();
        if (last) break;
#pragma unroll
        for (int c4 = 0; c4 < QC / 4; c4++) {
            float4 v = *reinterpret_cast<const float4*>(bvec + vec_pos(ch0) + 4 * c4);
            bw[4 * c4 + 0] = v.x;
            bw[4 * c4 + 1] = v.y;
            bw[4 * c4 + 2] = v.z;
            bw[4 * c4 + 3] = v.w;
        }
        // row step
        float rs[QR];
#pragma unroll
        for (int r = 0; r < QR; r++) {
            float s;
            if constexpr (KEEP_Y) {
                s = A[r][0] * bw[0];
#pragma unroll
                for (int c = 1; c < QC; c++) s = fmaf(A[r][c], bw[c], s);
            } else {
                s = mul_abs(A[r][0], bw[0]);
#pragma unroll
                for (int c = 1; c < QC; c++) s = fma_abs(A[r][c], bw[c], s);
            }
            rs[r] = s;
        }
        // Reduce-scatter over lane bits 0 and 1: lane (b0, b1) of a quad ends
        // with row 2 b0 + b1 summed over its quad, then over the remaining
        // channel-group bits; one reciprocal a lane, the four rows broadcast
        // back from their quad lanes.  Every add pairs the same two operands
        // as an all-reduce of each row would, so the sums are the same.
        const float r02 = rb0 ? rs[2] : rs[0], x02 = rb0 ? rs[0] : rs[2];
        const float r13 = rb0 ? rs[3] : rs[1], x13 = rb0 ? rs[1] : rs[3];
        const float t02 = r02 + i2f(__builtin_amdgcn_update_dpp(0, f2i(x02), 0xB1, 0xF, 0xF, true));
        const float t13 = r13 + i2f(__builtin_amdgcn_update_dpp(0, f2i(x13), 0xB1, 0xF, 0xF, true));
        const float tk = rb1 ? t13 : t02, tx = rb1 ? t02 : t13;
        float u = tk + i2f(__builtin_amdgcn_update_dpp(0, f2i(tx), 0x4E, 0xF, 0xF, true));
        u = xsum<3>(u);
        if constexpr (CGB >= 4) u = xsum<2>(u);
        if constexpr (CGB >= 5) u = xsum<4>(u);
        my_a = usable(u) ? __builtin_amdgcn_rcpf(u) : my_a;
        quad_bcast_rows(my_a, aw);
    }

    // ---- stage 4: per-token asymmetric round-to-nearest, packed in LDS ------
    float ic[QC];
#pragma unroll
    for (int c4 = 0; c4 < QC / 4; c4++) {
        float4 v = *reinterpret_cast<const float4*>(icvec + vec_pos(ch0) + 4 * c4);
        ic[4 * c4 + 0] = v.x;
        ic[4 * c4 + 1] = v.y;
        ic[4 * c4 + 2] = v.z;
        ic[4 * c4 + 3] = v.w;
    }
    uint8_t* img = smem;  // image of the record's code block
    // 2- and 4-bit codes: v_cvt_pk_u8_f32 rounds half to even, clamps to
    // [0, 255] and drops the byte into place; 6-bit codes: magic-number
    // rounding (x + 1.5 * 2^23 keeps rint(x) in the low mantissa bits).
    constexpr bool PKU8 = BITS != 6;
    uint32_t szk;  // fp16 scale and zero-point of row 2 b0 + b1 (quad lane b0 + 2 b1)
    // W = y / c, then u = (W - mn) / s, then (6-bit) the magic-rounded code
    // bits, all in place in the array that held y (or y^2 for D = 512)
    float (&u)[QR][QC] = *[&]() -> float(*)[QR][QC] {
        if constexpr (KEEP_Y) return &y; else return &A;
    }();
    {
        float mn[QR], mx[QR];
#pragma unroll
        for (int r = 0; r < QR; r++) {
#pragma unroll
            for (int c = 0; c < QC; c++) {
                float yv;
                if constexpr (KEEP_Y) {
                    yv = y[r][c];
                } else {
                    // y = sign(A) sqrt(|A|): v_sqrt_f32 (within 1 ulp), sign bit
                    // inserted with one v_bfi_b32
                    yv = __builtin_bit_cast(float, (fbits(__builtin_amdgcn_sqrtf(fabsf(A[r][c]))) & 0x7fffffffu) |
                                                       (fbits(A[r][c]) & 0x80000000u));
                }
                u[r][c] = yv * ic[c];
            }
            mn[r] = u[r][0];
            mx[r] = u[r][0];
#pragma unroll
            for (int c = 1; c < QC; c++) {
                mn[r] = fminf(mn[r], u[r][c]);
                mx[r] = fmaxf(mx[r], u[r][c]);
            }
        }
        // lane (b0, b1) of a quad ends with row 2 b0 + b1's minimum and maximum
        float mnk, mxk;
        row_minmax_scatter<CGB>(mn, mx, rb0, rb1, mnk, mxk);
        const float m0 = mnk + 0.0f;  // a zero row stores +0, not the -0 of a sign-flipped channel
        const float range = mxk - m0;
        const float sc = range * (1.0f / (float)QMAX);
        const float inv = range > 0.f ? (float)QMAX * __builtin_amdgcn_rcpf(range) : 0.f;
        const float nb = -m0 * inv;
        szk = float_to_half_bits(sc) | (float_to_half_bits(m0) << 16);
        float invr[QR], nbr[QR];
        quad_bcast_rows(inv, invr);
        quad_bcast_rows(nb, nbr);
#pragma unroll
        for (int r = 0; r < QR; r++) {
#pragma unroll
            for (int c = 0; c < QC; c++) {
                u[r][c] = fmaf(u[r][c], invr[r], nbr[r]);
                if constexpr (!PKU8) u[r][c] += kMagic;  // rint(u) in the low mantissa bits
            }
        }
    }
    auto fq = [&](int r, int c) -> uint32_t { return fbits(u[r][c]); };  // 6-bit: magic-rounded code
    // 4 codes -> bytes 0..3 of a dword
    auto pk4 = [](float a0, float a1, float a2, float a3) -> uint32_t {
        uint32_t v = __builtin_amdgcn_cvt_pk_u8_f32(a0, 0u, 0u);
        v = __builtin_amdgcn_cvt_pk_u8_f32(a1, 1u, v);
        v = __builtin_amdgcn_cvt_pk_u8_f32(a2, 2u, v);
        return __builtin_amdgcn_cvt_pk_u8_f32(a3, 3u, v);
    };
    // the statistics are done with the shared buffer (last barrier above);
    // the record's code image reuses it
    if constexpr (BYTE_IMAGE) {
        if constexpr (!CHMAJOR) {
            // token row t: codes of channels ch0 .. ch0 + 15 at bytes t D + ch0 ..
#pragma unroll
            for (int r = 0; r < QR; r++) {
                const float* x = u[r];
                *reinterpret_cast<uint4*>(img + (row0 + r) * D + ch0) =
                    make_uint4(pk4(x[0], x[1], x[2], x[3]), pk4(x[4], x[5], x[6], x[7]), pk4(x[8], x[9], x[10], x[11]),
                               pk4(x[12], x[13], x[14], x[15]));
            }
        } else {
            // channel row c of token block row0 / TB: codes of tokens row0 .. row0 + 3
#pragma unroll
            for (int c = 0; c < QC; c++)
                *reinterpret_cast<uint32_t*>(img + (row0 / TB) * (D * TB) + (ch0 + c) * TB + row0 % TB) =
                    pk4(u[0][c], u[1][c], u[2][c], u[3][c]);
        }
    } else if constexpr (!CHMAJOR) {
        // token-major: this lane's 16 codes of a row are contiguous
#pragma unroll
        for (int r = 0; r < QR; r++) {
            const float* x = u[r];
            uint8_t* dstp = img + ((row0 + r) * D + ch0) * BITS / 8;
            if constexpr (BITS == 4 && D == 128) {
                // unit (16 bytes) c of token row t sits at unit c ^ ((t >> 2) & 3)
                // of the row: the rows of lanes that differ in row-group bit 0
                // then use different bank quads
                const int t = row0 + r;
                dstp = img + t * 64 + ((((cg >> 1) ^ (t >> 2)) & 3) << 4) + 8 * (cg & 1);
            }
            if constexpr (BITS == 4) {
                // byte k = c_2k | c_2k+1 << 4
                const uint32_t e0 = pk4(x[0], x[2], x[4], x[6]), o0 = pk4(x[1], x[3], x[5], x[7]);
                const uint32_t e1 = pk4(x[8], x[10], x[12], x[14]), o1 = pk4(x[9], x[11], x[13], x[15]);
                *reinterpret_cast<uint2*>(dstp) = make_uint2(e0 | (o0 << 4), e1 | (o1 << 4));
            } else if constexpr (BITS == 2) {
                // byte k = c_4k | c_4k+1 << 2 | c_4k+2 << 4 | c_4k+3 << 6
                const uint32_t p0 = pk4(x[0], x[4], x[8], x[12]), p1 = pk4(x[1], x[5], x[9], x[13]);
                const uint32_t p2 = pk4(x[2], x[6], x[10], x[14]), p3 = pk4(x[3], x[7], x[11], x[15]);
                *reinterpret_cast<uint32_t*>(dstp) = p0 | (p1 << 2) | (p2 << 4) | (p3 << 6);
            } else {
                uint32_t g[4];
#pragma unroll
                for (int k = 0; k < 4; k++) g[k] = pack6x4(fq(r, 4 * k), fq(r, 4 * k + 1), fq(r, 4 * k + 2), fq(r, 4 * k + 3));
                uint32_t* d32 = reinterpret_cast<uint32_t*>(dstp);
                d32[0] = g[0] | (g[1] << 24);
                d32[1] = (g[1] >> 8) | (g[2] << 16);
                d32[2] = (g[2] >> 16) | (g[3] << 8);
            }
        }
    } else {
        // channel-major: this lane's 4 tokens of a channel are contiguous.
        // In the image, token block k (TB tokens) starts at k CM_BLK and
        // channel c's row of it at c TB BITS / 8 + 4 (c >> 4): 4 bytes of pad
        // after every 16 channels put the rows of the D/16 lanes that store
        // the same code position of their channels on different banks.
        constexpr int CM_BLK = D * TB * BITS / 8 + 4 * (D / 16);
        auto cm_at = [](int c, int t) {
            return (t / TB) * CM_BLK + c * (TB * BITS / 8) + 4 * (c >> 4) + (t % TB) * BITS / 8;
        };
        if constexpr (BITS == 2) {
            // byte of channel c = its 4 codes, token-ascending, 2 bits each
#pragma unroll
            for (int c4 = 0; c4 < QC / 4; c4++) {
                uint32_t p[QR];
#pragma unroll
                for (int r = 0; r < QR; r++) p[r] = pk4(u[r][4 * c4], u[r][4 * c4 + 1], u[r][4 * c4 + 2], u[r][4 * c4 + 3]);
                const uint32_t v = p[0] | (p[1] << 2) | (p[2] << 4) | (p[3] << 6);  // byte k: channel 4 c4 + k
#pragma unroll
                for (int k = 0; k < 4; k++) img[cm_at(ch0 + 4 * c4 + k, row0)] = (uint8_t)(v >> (8 * k));
            }
        } else if constexpr (BITS == 4) {
            // 16 bits of channel c: (c_t0 | c_t1 << 4) then (c_t2 | c_t3 << 4)
#pragma unroll
            for (int c4 = 0; c4 < QC / 4; c4++) {
                uint32_t p[QR];
#pragma unroll
                for (int r = 0; r < QR; r++) p[r] = pk4(u[r][4 * c4], u[r][4 * c4 + 1], u[r][4 * c4 + 2], u[r][4 * c4 + 3]);
                const uint32_t lo = p[0] | (p[1] << 4), hi = p[2] | (p[3] << 4);
                const uint32_t w01 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);  // channels 0, 1
                const uint32_t w23 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);  // channels 2, 3
                const int c0 = ch0 + 4 * c4;
                *reinterpret_cast<uint16_t*>(img + cm_at(c0, row0)) = (uint16_t)w01;
                *reinterpret_cast<uint16_t*>(img + cm_at(c0 + 1, row0)) = (uint16_t)(w01 >> 16);
                *reinterpret_cast<uint16_t*>(img + cm_at(c0 + 2, row0)) = (uint16_t)w23;
                *reinterpret_cast<uint16_t*>(img + cm_at(c0 + 3, row0)) = (uint16_t)(w23 >> 16);
            }
        } else {
#pragma unroll
            for (int c = 0; c < QC; c++) {
                const uint32_t v = pack6x4(fq(0, c), fq(1, c), fq(2, c), fq(3, c));
                uint8_t* d8 = img + cm_at(ch0 + c, row0);
                d8[0] = (uint8_t)v;
                d8[1] = (uint8_t)(v >> 8);
                d8[2] = (uint8_t)(v >> 16);
            }
        }
    }
    // per-token scale and zero-point: the quad of channel groups 0..3 holds
    // the row group's 4 tokens, one each
    if (cg < 4) {
        *reinterpret_cast<uint32_t*>(rec + CODE_BYTES + 4 * (row0 + 2 * (int)rb0 + (int)rb1)) = szk;
    }
    // column scales, normalized basis
    if (tid < D / 8) {
        *reinterpret_cast<uint4*>(rec + CODE_BYTES + 4 * T + 16 * tid) =
            *reinterpret_cast<const uint4*>(cvec + 8 * tid);
    }
    __syncthreads();

    // ---- stage 5: the code image leaves in 16-byte stores -------------------
    if constexpr (BITS == 3 || BITS == 5) {
        // every 32 consecutive codes of the byte image become BITS dwords of
        // the LSB-first stream; all groups are read before any is written back
        constexpr int NG = T * D / 32;
        static_assert(NG % NT == 0, "whole groups per thread");
        constexpr int GPT = NG / NT;
        constexpr uint32_t M = (1u << BITS) - 1;
        // 4 codes (bytes of d) -> 4 BITS bits
        auto pack4 = [](uint32_t d) -> uint32_t {
            return (d & M) | ((d >> (8 - BITS)) & (M << BITS)) | ((d >> (16 - 2 * BITS)) & (M << (2 * BITS))) |
                   ((d >> (24 - 3 * BITS)) & (M << (3 * BITS)));
        };
        uint32_t words[GPT][BITS];
#pragma unroll
        for (int k = 0; k < GPT; k++) {
            const int g = tid + k * NT;
            const uint4 a = reinterpret_cast<const uint4*>(img)[2 * g];
            const uint4 b = reinterpret_cast<const uint4*>(img)[2 * g + 1];
            const uint32_t d[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
            uint64_t acc = 0;
            int nb = 0, o = 0;
#pragma unroll
            for (int i = 0; i < 8; i++) {
                acc |= (uint64_t)pack4(d[i]) << nb;
                nb += 4 * BITS;
                if (nb >= 32) {
                    words[k][o++] = (uint32_t)acc;
                    acc >>= 32;
                    nb -= 32;
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < GPT; k++) {
            uint32_t* dst = reinterpret_cast<uint32_t*>(img) + BITS * (tid + k * NT);
#pragma unroll
            for (int o = 0; o < BITS; o++) dst[o] = words[k][o];
        }
        __syncthreads();
    }
    if constexpr (BYTE_IMAGE) {
        uint4* dst4 = reinterpret_cast<uint4*>(rec);
        for (int u = tid; u < CODE_BYTES / 16; u += NT) dst4[u] = reinterpret_cast<const uint4*>(img)[u];
    } else {
        // thread tid moves units tid, tid + NT, ...: consecutive lanes read
        // consecutive LDS units and write consecutive 16-byte chunks
        constexpr int UNITS = CODE_BYTES / 16 / NT;   // BITS / 2 units per thread
        uint4* dst4 = reinterpret_cast<uint4*>(rec);
#pragma unroll
        for (int k = 0; k < UNITS; k++) {
            const int u = tid + k * NT;
            if constexpr (CHMAJOR) {
                // unit u lies in token block 16 u / RBLK, channel row o / (TB BITS / 8)
                // of it (rows are 16-byte multiples), shifted by the block's and
                // the row's pads: 4-byte aligned
                constexpr int RROW = TB * BITS / 8, RBLK = D * RROW, CM_BLK = RBLK + 4 * (D / 16);
                static_assert(RROW % 16 == 0, "channel rows of whole 16-byte units");
                const int blk = 16 * u / RBLK, o = 16 * u - blk * RBLK;
                const uint32_t* p = reinterpret_cast<const uint32_t*>(img + blk * CM_BLK + o + 4 * ((o / RROW) >> 4));
                dst4[u] = make_uint4(p[0], p[1], p[2], p[3]);
            } else {
                int pu = u;
                if constexpr (BITS == 4 && D == 128) pu = (u & ~3) | ((u ^ (u >> 4)) & 3);  // row t = u >> 2
                dst4[u] = reinterpret_cast<const uint4*>(img)[pu];
            }
        }
    }
}

// One launch quantizes keys and values (or the MLA latent): workgroup
// 2*(i*H + h) + kind takes page i, head h, kind 0 = keys (token-major codes),
// kind 1 = values (channel-major codes).
template <int D, int T, int KB, int VB, bool HASV>
// D = 128: three waves per SIMD (168 VGPRs; the rotation's MFMA accumulators
// and the rows it fills peak there); a D = 512 workgroup is itself four
// waves per SIMD
__global__ void __launch_bounds__(T * D / 64, D == 128 ? 3 : 4)
quantize_kernel(const uint16_t* __restrict__ kpool, const uint16_t* __restrict__ vpool,
                uint8_t* __restrict__ krec, uint8_t* __restrict__ vrec, const int32_t* __restrict__ src,
                const int32_t* __restrict__ dst, int32_t H, int64_t n_fpages, int64_t n_qpages, int32_t n_iters) {
    using S = TileShape<D, T>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[S::SMEM];
    __shared__ __attribute__((aligned(16))) float vec[VecShape<D>::FLOATS];
    const int kind = HASV ? (int)(wg_x() & 1u) : 0;
    const int r = HASV ? (int)(wg_x() >> 1) : (int)wg_x();
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

// Keys or values alone (code widths outside 2, 4, 6 pair through two of
// these launches): workgroup i*H + h takes page i, head h.
template <int D, int T, int BITS, bool CHMAJOR>
__global__ void __launch_bounds__(T * D / 64, D == 128 ? 3 : 4)
quantize_one_kernel(const uint16_t* __restrict__ pool, uint8_t* __restrict__ recs, const int32_t* __restrict__ src,
                    const int32_t* __restrict__ dst, int32_t H, int64_t n_fpages, int64_t n_qpages, int32_t n_iters) {
    using S = TileShape<D, T>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[S::SMEM];
    __shared__ __attribute__((aligned(16))) float vec[VecShape<D>::FLOATS];
    const int r = (int)wg_x();
    const int i = r / H;
    const int h = r - i * H;
    const int sp = src[i];
    const int dp = dst[i];
    if (sp < 0 || (int64_t)sp >= n_fpages || dp < 0 || (int64_t)dp >= n_qpages) return;
    constexpr int REC = T * D * BITS / 8 + 4 * T + 2 * D;
    quantize_tile<D, T, BITS, CHMAJOR>(pool + ((int64_t)sp * H + h) * (int64_t)(T * D),
                                       recs + ((int64_t)dp * H + h) * REC, smem, vec, n_iters);
}

}  // namespace

template <int D, int T, int BITS, bool CHMAJOR>
hipError_t launch_quantize_one(const QuantizeArgs& a, hipStream_t st) {
    const int64_t blocks = (int64_t)a.n * a.H;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((quantize_one_kernel<D, T, BITS, CHMAJOR>), dim3((unsigned)blocks), dim3(T * D / 64), 0, st,
                       static_cast<const uint16_t*>(CHMAJOR ? a.v_fp16 : a.k_fp16),
                       static_cast<uint8_t*>(CHMAJOR ? a.v_records : a.k_records), a.src, a.dst, a.H, a.n_fpages,
                       a.n_qpages, a.n_iters);
    return hipGetLastError();
}

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
    template hipError_t launch_quantize_shape<D, 64, 6, 6, true>(const QuantizeArgs&, hipStream_t);  \
    KVARN_QUANTIZE_ONE_T(D, 128)                                                                 \
    KVARN_QUANTIZE_ONE_T(D, 64)
#define KVARN_QUANTIZE_ONE_T(D, T)                                                               \
    KVARN_QUANTIZE_ONE_B(D, T, 2) KVARN_QUANTIZE_ONE_B(D, T, 3) KVARN_QUANTIZE_ONE_B(D, T, 4)    \
    KVARN_QUANTIZE_ONE_B(D, T, 5) KVARN_QUANTIZE_ONE_B(D, T, 6) KVARN_QUANTIZE_ONE_B(D, T, 8)
#define KVARN_QUANTIZE_ONE_B(D, T, B)                                                            \
    template hipError_t launch_quantize_one<D, T, B, false>(const QuantizeArgs&, hipStream_t);    \
    template hipError_t launch_quantize_one<D, T, B, true>(const QuantizeArgs&, hipStream_t);

}  // namespace kvarn
