// KVarN paged GQA decode attention for gfx950: split-K partials + combine.
//
// The records are never dequantized to memory (evermx.com KVarN review,
// method paragraph: scales folded back in at read time).  With the rotated
// query q' = H q / sqrt(D) and, per record, the column scales C, per-token
// scale S_t and zero-point Zp_t:
//   score_t  = <q, k_t> = S_t <q' * C, code_t> + Zp_t * sum(q' * C)
//   sum_t p_t v_t = H ( C_V * ( sum_t (p_t S_t) code_t + sum_t p_t Zp_t ) ) / sqrt(D)
// so each split accumulates the value sum in the rotated basis and the
// combine applies H once.  fp16 sink and tail pages (gmlx "KV cache
// quantization", "The two schemes") are accumulated in the original basis
// into a second sum that the combine adds after the rotation.
//
// Both contractions of a quantized page run on the 4x4x4 fp16 MFMA with 16
// blocks: the four query heads of a KV head are its 4 rows, and one operand
// is broadcast from one block to all 16 (CBSZ = 4, ABID = the block), so a
// wave covers 64 tokens (scores, lane = token) or 64 channels (values,
// lane = channel) per instruction.  A B-bit code c enters the MFMA as the
// fp16 number 1 + c / 2^B, made by or-ing the code into the mantissa of 1.0;
// the constant part is taken back out with sum(q' * C) and sum(p (Zp - 2^B S)).
// The other operand (a query, the query times C, or the weights times S) is
// split into fp16 high and low parts, two MFMAs on the same codes, so the
// products keep fp32 accuracy.
//
// One wave per workgroup per (split, KV head, sequence); split s visits pages
// s, s + nsplit, ..., so the fp16 pages at both ends spread over the splits,
// 64 tokens per step; the next step's codes and scales load during the
#pragma once

// current one.
#include <math.h>

#include <utility>

#include "decode_combine.hpp"
#include "kvarn_device.hpp"
#include "kvarn_internal.hpp"

namespace kvarn {
namespace {

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// 4x4x4 fp16 MFMA with 16 blocks, operand A broadcast from block ABID
template <int ABID>
__device__ __forceinline__ f4 mfma_bcast(h4 a, h4 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_4x4x4f16(a, b, c, 4, ABID, 0);
}
// the same with broadcast groups of 8 blocks: blocks 0-7 (lanes 0-31) take
// operand A from block ABID, blocks 8-15 (lanes 32-63) from block 8 + ABID
template <int ABID>
__device__ __forceinline__ f4 mfma_bcast8(h4 a, h4 b, f4 c) {
    static_assert(ABID < 8, "source block inside the group");
    return __builtin_amdgcn_mfma_f32_4x4x4f16(a, b, c, 3, ABID, 0);
}

template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
// f(integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---- packed codes as MFMA operands ----------------------------------------
// The 4 k-slots of operand i hold codes code_of<B>(i, k) of an LSB-first
// stream.  For B = 2 and 4 a 32-bit word holds codes s and s + 16/B in its
// two 16-bit halves, so a pair is one shift and one and-or; the k order
// follows the pairs.  6-bit codes are taken in stream order.
template <int B>
__host__ __device__ constexpr int code_of(int i, int k) {
    if constexpr (B == 4) return 8 * (i >> 1) + 2 * (i & 1) + (k >> 1) + 4 * (k & 1);
    else if constexpr (B == 2) return 16 * (i >> 2) + 2 * (i & 3) + (k >> 1) + 8 * (k & 1);
    else return 4 * i + k;
}

// position 4 i + k of stream code n (inverse of code_of)
template <int B>
__device__ __forceinline__ int pos_of(int n) {
    if constexpr (B == 4) {
        const int u = n & 7;
        return 4 * (2 * (n >> 3) + ((u & 3) >> 1)) + (((u & 1) << 1) | (u >> 2));
    } else if constexpr (B == 2) {
        const int u = n & 15;
        return 4 * (4 * (n >> 4) + ((u & 7) >> 1)) + (((u & 1) << 1) | (u >> 3));
    } else {
        return n;
    }
}

// fp16 pair (1 + c_s / 2^B, 1 + c_{s + 16/B} / 2^B) from word w, B = 2 or 4
template <int B>
__device__ __forceinline__ uint32_t code_pair(uint32_t w, int s) {
    constexpr uint32_t mask = B == 4 ? 0x03C003C0u : 0x03000300u;
    const int sh = (10 - B) - B * s;  // code s to mantissa bits 10-B .. 9
    const uint32_t v = sh >= 0 ? (w << sh) : (w >> -sh);
    return (v & mask) | 0x3C003C00u;
}

// operand i (4 codes, as 1 + c / 2^B) from the words w[] of a stream segment
template <int B>
__device__ __forceinline__ h4 code_operand(const uint32_t* w, int i) {
    uint32_t lo, hi;
    if constexpr (B == 4) {
        const uint32_t x = w[i >> 1];
        lo = code_pair<4>(x, 2 * (i & 1));
        hi = code_pair<4>(x, 2 * (i & 1) + 1);
    } else if constexpr (B == 2) {
        const uint32_t x = w[i >> 2];
        lo = code_pair<2>(x, 2 * (i & 3));
        hi = code_pair<2>(x, 2 * (i & 3) + 1);
    } else if constexpr (B != 6) {
        // widths 3, 5, 8: stream order, operand i = codes 4 i .. 4 i + 3 at
        // bits 4 B i .. 4 B i + 4 B - 1 (i is a compile-time constant at every use)
        constexpr uint32_t M = (1u << B) - 1;
        const int bit = 4 * B * i;
        const int j = bit >> 5, o = bit & 31;
        const uint32_t f = o + 4 * B <= 32 ? (w[j] >> o) : __builtin_amdgcn_alignbit(w[j + 1], w[j], o);
        // code k to mantissa bits 10 - B .. 9 of half k & 1 of word k >> 1
        auto place = [&](int k) -> uint32_t {
            const int from = B * k, to = (10 - B) + 16 * (k & 1);
            const uint32_t v = to >= from ? (f << (to - from)) : (f >> (from - to));
            return v & (M << to);
        };
        lo = place(0) | place(1) | 0x3C003C00u;
        hi = place(2) | place(3) | 0x3C003C00u;
    } else {
        // 16 codes in 3 words; operand i takes bits 24 (i & 3) .. +23 of group i >> 2
        const int g = 3 * (i >> 2), e = i & 3;
        const int bit = 24 * e;
        const uint32_t f = (bit & 31) + 24 <= 32 ? (w[g + (bit >> 5)] >> (bit & 31))
                                                : __builtin_amdgcn_alignbit(w[g + (bit >> 5) + 1], w[g + (bit >> 5)], bit & 31);
        lo = ((f << 4) & 0x3F0u) | ((f << 14) & 0x03F00000u) | 0x3C003C00u;
        hi = ((f >> 8) & 0x3F0u) | ((f << 2) & 0x03F00000u) | 0x3C003C00u;
    }
    return __builtin_bit_cast(h4, make_uint2(lo, hi));
}

__device__ __forceinline__ void load_words(uint32_t* w, const uint8_t* p, int nbytes16) {
#pragma unroll
    for (int k = 0; k < nbytes16; k++) {
        const uint4 v = reinterpret_cast<const uint4*>(p)[k];
        w[4 * k] = v.x; w[4 * k + 1] = v.y; w[4 * k + 2] = v.z; w[4 * k + 3] = v.w;
    }
}

// NW words from p: 16-byte loads when NW is a multiple of 4, else 8-byte ones
// (segments of odd code widths are 8-byte aligned)
template <int NW>
__device__ __forceinline__ void load_seg(uint32_t* w, const uint8_t* p) {
    if constexpr (NW % 4 == 0) {
        load_words(w, p, NW / 4);
    } else {
        static_assert(NW % 2 == 0, "whole 8-byte units");
#pragma unroll
        for (int k = 0; k < NW / 2; k++) {
            const uint2 v = reinterpret_cast<const uint2*>(p)[k];
            w[2 * k] = v.x;
            w[2 * k + 1] = v.y;
        }
    }
}

// sum over the 16 lanes of one residue class mod 4 within each 32-lane half
__device__ __forceinline__ float sum_blocks_half(float v) {
    v += i2f(__builtin_amdgcn_update_dpp(0, f2i(v), 0x124, 0xF, 0xF, true));  // row_ror 4
    v += i2f(__builtin_amdgcn_update_dpp(0, f2i(v), 0x128, 0xF, 0xF, true));  // row_ror 8
    v += xor_lane<4>(v);
    return v;
}

// fp16 sink and tail pages (gmlx "KV cache quantization", "The two
// schemes"): workgroups of the split kernels' grid past the splits, one wave
// per (fp16 slot f, group h of 4 query heads, query row); the group's KV head
// is h / GS.  Slot f is the 64-token part f % (T /
// 64) of the (f / (T / 64))-th fp16 page of the sequence (sink pages, then
// tail pages); its partial goes to split nsplit + f with a zero rotated-basis
// sum.  Scores on the MFMA with the plain query (fp16 high and low parts),
// lane = token; value sums on the VALU, D/8 lanes per token row.
//
// Key rows are read so that both 64-byte halves of every 128-byte line are
// requested by one load instruction: a line whose halves are requested by
// different instructions, the second while the fill of the first is still
// pending, is fetched from HBM twice (about 2x the key bytes, measured
// with the L2's read-request counters).  Tokens t and 32 + t pair up: one
// load gives lane t (< 32) piece p of token t and lane 32 + t piece p + 4 of
// token t, the next gives lane t piece p + 4 of token 32 + t and lane 32 + t
// piece p of token 32 + t.  Each lane accumulates what it holds: the lower
// and the upper lane halves hold different channel groups in one register,
// so the MFMA broadcasts its query operand within groups of 8 blocks, with
// the query slots held a second time, half-swapped, for the second load.
// The first load's sums of lanes t and 32 + t make token t's score, the
// second load's those of token 32 + t: one v_permlane32_swap per head adds
// them up at the end.
template <int D, int T>
__device__ __forceinline__ void fp16_block(const DecodeArgs& a, const int f, const int h, const int b,
                                           float4* pf /* LDS, 64 entries: weights of the part */) {
    constexpr int G = 4;
    constexpr int NS = D / 64;
    constexpr int NC = D / 128;
    constexpr int TS = T / 64;
    constexpr int WS = D + 4;           // partial: m, l, pad, pad, value sums

    const int lane = threadIdx.x & 63;  // workgroups of head_dim 512 hold two waves
    const int blk = lane >> 2, m = lane & 3;
    const int Hq = a.Hq;
    const float sm2 = a.sm_scale * kLog2e;
    const int bs = b / a.M;  // sequence of query row b
    const int L = min(a.seq_lens[bs], a.max_pages * T);
    const int A = attend_len(a, b, L, a.max_pages * T);  // tokens this row attends
    const int npages = A > 0 ? (A + T - 1) / T : 0;
    const int nq = (L - a.sink - a.tail >= T) ? (L - a.sink - a.tail) / T : 0;
    const int sp = a.sink / T;
    const int fpg = f / TS, sb = f % TS;
    const int page = fpg < sp ? fpg : sp + nq + (fpg - sp);
    int id = -1;
    int nvalid = 0;  // valid tokens of the part
    if (page < npages) {
        nvalid = min(64, min(T, A - page * T) - 64 * sb);
        id = a.block_table[(int64_t)bs * a.max_pages + page];
        if (id < 0 || (int64_t)id >= a.n_fpages || nvalid <= 0) id = -1;
    }

    constexpr int LPT = D / 8;     // lanes per token row in the value sums
    constexpr int TG = 64 / LPT;   // tokens per load instruction
    float mx[G], lsum[G], accp[8][G];
#pragma unroll
    for (int g = 0; g < G; g++) {
        mx[g] = -INFINITY;
        lsum[g] = 0.f;
#pragma unroll
        for (int c = 0; c < 8; c++) accp[c][g] = 0.f;
    }
    if (id >= 0) {  // uniform
        // the plain query (fp16 high and low parts) at this lane's operand
        // slots: 4 consecutive channels 4 i .. 4 i + 3 per slot
        float qx[NS][4];
        const int64_t qrow = ((int64_t)b * Hq + h * G + m) * D;
#pragma unroll
        for (int r = 0; r < NS; r++) q_load<4>(a.q, a.q_dtype, qrow + 4 * (32 * (r >> 1) + blk + 16 * (r & 1)), qx[r]);
        h4 qp[NS], qpl[NS];
#pragma unroll
        for (int r = 0; r < NS; r++)
#pragma unroll
            for (int kk = 0; kk < 4; kk++) {
                qp[r][kk] = (_Float16)qx[r][kk];
                qpl[r][kk] = (_Float16)(qx[r][kk] - (float)qp[r][kk]);
            }
        // the same slots half-swapped: lane l holds what lane l ^ 32 holds
        // above, i.e. block blk the channel group of block blk ^ 8
        const bool upper = lane >= 32;
        auto half_swap = [&](h4 v) {
            uint2 w = __builtin_bit_cast(uint2, v);
            const auto x = __builtin_amdgcn_permlane32_swap(w.x, w.x, false, false);
            const auto y = __builtin_amdgcn_permlane32_swap(w.y, w.y, false, false);
            // x[0]: lower half of w.x in both halves; x[1]: upper half of w.x in both
            return __builtin_bit_cast(h4, make_uint2(upper ? x[0] : x[1], upper ? y[0] : y[1]));
        };
        h4 qps[NS], qpls[NS];
#pragma unroll
        for (int r = 0; r < NS; r++) {
            qps[r] = half_swap(qp[r]);
            qpls[r] = half_swap(qpl[r]);
        }
        float s[G];
        {
            // token 0 of the part; a 16-byte piece p holds channels 8 p .. 8 p + 7
            const uint16_t* kt = static_cast<const uint16_t*>(a.k_fp16) + (((int64_t)id * a.H + h / a.GS) * T + 64 * sb) * D;
            const int t5 = lane & 31;
            const int hx = upper ? 4 : 0;  // piece offset of the first load in this lane half
            const f4 zero = {0.f, 0.f, 0.f, 0.f};
            f4 ax0 = zero, ax1 = zero, ay0 = zero, ay1 = zero;
#pragma unroll
            for (int c = 0; c < NC; c++) {
                // pieces pa and pa + 4 (the two halves of a 128-byte line) of a
                // 256-byte chunk of 128 channels
                static_for<8>([&](auto jc) {
                    constexpr int j = decltype(jc)::value;
                    constexpr int pa = (j & 3) + 8 * (j >> 2);
                    // x: tokens 0-31, piece pa (lower lanes) or pa + 4 (upper);
                    // y: tokens 32-63, piece pa + 4 (lower lanes) or pa (upper)
                    const uint4 x = *reinterpret_cast<const uint4*>(kt + (int64_t)t5 * D + 128 * c + 8 * (pa + hx));
                    const uint4 y = *reinterpret_cast<const uint4*>(kt + (int64_t)(32 + t5) * D + 128 * c + 8 * (pa + 4 - hx));
                    const h4 x0 = __builtin_bit_cast(h4, make_uint2(x.x, x.y));
                    const h4 x1 = __builtin_bit_cast(h4, make_uint2(x.z, x.w));
                    const h4 y0 = __builtin_bit_cast(h4, make_uint2(y.x, y.y));
                    const h4 y1 = __builtin_bit_cast(h4, make_uint2(y.z, y.w));
                    // channel group 2 pa + e of the chunk (lower lanes of x): slot
                    // r, block ab + e; the upper lanes' group is 8 higher, block 8 + ab + e
                    constexpr int ab = (2 * pa) & 15;
                    const int r = 2 * c + (pa >> 3);
                    ax0 = mfma_bcast8<ab>(qp[r], x0, ax0);
                    ax1 = mfma_bcast8<ab>(qpl[r], x0, ax1);
                    ax0 = mfma_bcast8<ab + 1>(qp[r], x1, ax0);
                    ax1 = mfma_bcast8<ab + 1>(qpl[r], x1, ax1);
                    ay0 = mfma_bcast8<ab>(qps[r], y0, ay0);
                    ay1 = mfma_bcast8<ab>(qpls[r], y0, ay1);
                    ay0 = mfma_bcast8<ab + 1>(qps[r], y1, ay0);
                    ay1 = mfma_bcast8<ab + 1>(qpls[r], y1, ay1);
                });
            }
            // lane t < 32: x sums of lanes t and t + 32 (token t); lane t + 32: y sums (token t + 32)
            const f4 X = ax0 + ax1, Y = ay0 + ay1;
            f4 R;
#pragma unroll
            for (int g = 0; g < G; g++) {
                const auto w = __builtin_amdgcn_permlane32_swap((unsigned)f2i(X[g]), (unsigned)f2i(Y[g]), false, false);
                R[g] = i2f((int)w[0]) + i2f((int)w[1]);
            }
            const bool valid = lane < nvalid;
#pragma unroll
            for (int g = 0; g < G; g++) s[g] = valid ? sm2 * R[g] : -INFINITY;
        }
        // softmax over the part: its first token is valid
        float p[G];
#pragma unroll
        for (int g = 0; g < G; g++) {
            mx[g] = wave_max_all(s[g]);
            p[g] = exp2f(s[g] - mx[g]);
            lsum[g] += p[g];
        }
        pf[lane] = make_float4(p[0], p[1], p[2], p[3]);
        wave_sync();
        // value sums: D/8 lanes per token row (16-byte loads of 8 channels), TG
        // tokens per load instruction, the token groups summed at the end
        const uint16_t* vp = static_cast<const uint16_t*>(a.v_fp16) + (((int64_t)id * a.H + h / a.GS) * T + 64 * sb) * D;
        const int tg = lane / LPT, cc = lane % LPT;
        // branch-free: a token past the end has weight 0 (its score is
        // -inf) and reads the last valid token's values instead of its own
#pragma unroll 8
        for (int tt = 0; tt < 64; tt += TG) {
            const int t = tt + tg;
            const uint4 w = *reinterpret_cast<const uint4*>(vp + (int64_t)min(t, nvalid - 1) * D + 8 * cc);
            const float4 pv = pf[t];
            const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int kk = 0; kk < 8; kk++) {
                const float v = half_bits_to_float((ww[kk >> 1] >> (16 * (kk & 1))) & 0xffffu);
                accp[kk][0] = fmaf(pv.x, v, accp[kk][0]);
                accp[kk][1] = fmaf(pv.y, v, accp[kk][1]);
                accp[kk][2] = fmaf(pv.z, v, accp[kk][2]);
                accp[kk][3] = fmaf(pv.w, v, accp[kk][3]);
            }
        }
    }
    // sum the token groups (lane bits above log2(LPT))
#pragma unroll
    for (int kk = 0; kk < 8; kk++)
#pragma unroll
        for (int g = 0; g < G; g++) {
            float v = accp[kk][g];
            if constexpr (TG >= 4) v += xor_lane<4>(v);
            if constexpr (TG >= 2) v += lane_bcast32(v);
            accp[kk][g] = v;
        }
    float* wsp = a.ws + (int64_t)a.B * Hq * D;
#pragma unroll
    for (int g = 0; g < G; g++) {
        const float lt = wave_sum_all(lsum[g]);
        float* o = wsp + (((int64_t)b * Hq + h * G + g) * (a.nsplit + a.nfsplit) + a.nsplit + f) * WS;
        if (lane == 0) {
            o[0] = mx[g];
            o[1] = lt;
        }
        if (lane < LPT) {
#pragma unroll
            for (int c = 0; c < 8; c++) o[4 + 8 * lane + c] = accp[c][g];
        }
    }
}

// exponent e of x = f 2^e with 0.5 <= |f| < 1 (0 for x = 0)
__device__ __forceinline__ int frexp_exp(float x) { return __builtin_amdgcn_frexp_expf(x); }

// Reductions of four values per lane (one per query head) over the 64 lanes,
// returned wave-uniform.  Inside each 16-lane row: fused DPP (xor 1, xor 2,
// rotate 4, rotate 8); across rows the heads are paired, so one
// v_permlane16_swap serves heads 0/1 (and 2/3) and one v_permlane32_swap
// serves all four: afterwards row r holds head r's result, read from lane 16 r.
#define KVARN_DPP4(OP, CTRL)                                                                  \
    asm volatile("s_nop 1\n\t"                                                                 \
                 OP "_dpp %0, %0, %0 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                 \
                 OP "_dpp %1, %1, %1 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                 \
                 OP "_dpp %2, %2, %2 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                 \
                 OP "_dpp %3, %3, %3 " CTRL " row_mask:0xf bank_mask:0xf"                     \
                 : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]))

template <bool MAX>
__device__ __forceinline__ void wave_reduce4(float (&v)[4], float (&out)[4]) {
    if constexpr (MAX) {
        KVARN_DPP4("v_max_f32", "quad_perm:[1,0,3,2]");
        KVARN_DPP4("v_max_f32", "quad_perm:[2,3,0,1]");
        KVARN_DPP4("v_max_f32", "row_ror:4");
        KVARN_DPP4("v_max_f32", "row_ror:8");
    } else {
        KVARN_DPP4("v_add_f32", "quad_perm:[1,0,3,2]");
        KVARN_DPP4("v_add_f32", "quad_perm:[2,3,0,1]");
        KVARN_DPP4("v_add_f32", "row_ror:4");
        KVARN_DPP4("v_add_f32", "row_ror:8");
    }
    auto op = [](float x, float y) { return MAX ? fmaxf(x, y) : x + y; };
    const auto p01 = __builtin_amdgcn_permlane16_swap((unsigned)f2i(v[0]), (unsigned)f2i(v[1]), false, false);
    const auto p23 = __builtin_amdgcn_permlane16_swap((unsigned)f2i(v[2]), (unsigned)f2i(v[3]), false, false);
    const float m01 = op(i2f((int)p01[0]), i2f((int)p01[1]));  // rows 0, 2: head 0; rows 1, 3: head 1
    const float m23 = op(i2f((int)p23[0]), i2f((int)p23[1]));  // rows 0, 2: head 2; rows 1, 3: head 3
    const auto q = __builtin_amdgcn_permlane32_swap((unsigned)f2i(m01), (unsigned)f2i(m23), false, false);
    const float r = op(i2f((int)q[0]), i2f((int)q[1]));        // row g: head g
#pragma unroll
    for (int g = 0; g < 4; g++) out[g] = i2f(__builtin_amdgcn_readlane(f2i(r), 16 * g));
}

// Waves per (split, KV head, sequence) of decode_split_kernel: one per 128
// channels, the partial scores summed through LDS once per step, so that a
// whole step's codes are prefetched in the registers of three waves per SIMD.
template <int D>
constexpr int split_waves() { return D / 128; }

template <int D, int T, int KB, int VB>
__global__ void __launch_bounds__(64 * split_waves<D>(), 3) decode_split_kernel(DecodeArgs a) {
    constexpr int G = 4;
    constexpr int NWV = split_waves<D>();
    constexpr int DH = D / NWV;           // channels of one wave
    constexpr int NS = DH / 64;           // operand slots per lane; value channel sets
    constexpr int NC = DH / 128;          // 128-channel chunks of a key row
    constexpr int TS = T / 64;            // 64-token sub-blocks of a page
    constexpr int KCB = T * D * KB / 8;
    constexpr int VCB = T * D * VB / 8;
    constexpr int KREC = KCB + 4 * T + 2 * D;
    constexpr int VREC = VCB + 4 * T + 2 * D;
    constexpr int KROW = D * KB / 8;      // code bytes of one token
    constexpr int KCH = 128 * KB / 8;     // code bytes of a 128-channel chunk
    constexpr int VROW = T * VB / 8;      // code bytes of one channel
    constexpr int WS = D + 4;           // partial: m, l, pad, pad, value sums
    constexpr float FK = (float)(1 << KB), FV = (float)(1 << VB);
    static_assert(KCH % 16 == 0 && VROW % 8 == 0, "16-byte key chunks, 8-byte value rows");

    __shared__ __attribute__((aligned(16))) _Float16 pt[NWV][2][G][64];  // p * S_V of a step (high, low), by operand position
    __shared__ float4 pf[NWV][64];
    __shared__ float xs[NWV > 1 ? 2 : 1][NWV][G][64];  // partial scores by step parity

    const int wave = NWV > 1 ? __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) : 0;
    const int lane = threadIdx.x & 63;
    // grid z < B: quantized-page splits; z >= B: fp16 page slots (one per
    // wave), dispatched after every split so that they fill the splits' tail
    if ((int)blockIdx.z >= a.B) {
        const int slot = (int)blockIdx.x * NWV + wave;
        if (slot < a.nfsplit) fp16_block<D, T>(a, slot, blockIdx.y, blockIdx.z - a.B, pf[wave]);
        return;
    }
    if ((int)blockIdx.x >= a.nsplit) return;
    // h: group of 4 query heads 4 h .. 4 h + 3, of KV head kvh (G / 4 groups per KV head)
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z, kvh = h / a.GS;
    const int blk = lane >> 2, m = lane & 3;  // MFMA block; row (query head) of the broadcast operand
    const int Hq = a.Hq;
    const float sm2 = a.sm_scale * kLog2e;

    // rotated query (fp32) at the channels of this lane's operand slots.
    // Slot r serves operand 32 (r >> 1) + blk + 16 (r & 1) of the wave's
    // channels, operand DH / 4 * wave + ... of the row.
    const float* qr = a.ws + ((int64_t)b * Hq + h * G + m) * D;
    float qv[NS][4];
#pragma unroll
    for (int r = 0; r < NS; r++) {
        const int i = 32 * (r >> 1) + blk + 16 * (r & 1) + (DH / 4) * wave;
#pragma unroll
        for (int k = 0; k < 4; k++) qv[r][k] = qr[code_of<KB>(i, k)];
    }

    const int bs = b / a.M;  // sequence of query row b (its quantized pages lie before every query token)
    const int L = min(a.seq_lens[bs], a.max_pages * T);
    const int nq = (L - a.sink - a.tail >= T) ? (L - a.sink - a.tail) / T : 0;
    const int sp = a.sink / T;

    float mrun[G], lp[G], accr[NS][G];
#pragma unroll
    for (int g = 0; g < G; g++) {
        mrun[g] = -INFINITY;
        lp[g] = 0.f;
#pragma unroll
        for (int s = 0; s < NS; s++) accr[s][g] = 0.f;
    }

    // Steps: the 64-token halves h of this split's pages (pages split,
    // split + nsplit, ...), in order.  A quantized step's key words (chunk 0),
    // scale words and, on a page's first half, column scales are loaded during
    // the previous step: the key part once that step's scores have consumed
    // theirs, the value part once its value sums have.
    constexpr int KW = KCH / 4;           // words of one 128-channel key chunk
    constexpr int VRW = VROW / 4;         // value code words of one channel (whole page)
    constexpr int VHW = 64 * VB / 32;     // value code words of one channel over 64 tokens
    // (8-bit codes, 32 words, load inside the step: prefetching them too
    // spills registers)
    constexpr bool PREK = KW <= 24;
    // the wave's key chunk prefetched one step ahead
    constexpr int NKP = 1;
    // the wave's value words of a step prefetched one step ahead (24 words at most)
    constexpr bool PREV = NS * VHW <= 24;
    static_assert(VRW == TS * VHW, "a channel row is TS halves");
    // value codes of channel c over the 64 tokens of step half hh: records
    // keep values in 64-token blocks, each channel's 64 codes in a row, so a
    // step reads one contiguous run of the record
    auto vseg = [](int hh, int c) -> int64_t { return (int64_t)hh * (64 * D * VB / 8) + (int64_t)c * (8 * VB); };
    const int npg = nq > split ? (nq - split + a.nsplit - 1) / a.nsplit : 0;  // quantized pages of this split
    const int nst = npg * TS;
    const uint8_t* const krec = static_cast<const uint8_t*>(a.k_records);
    const uint8_t* const vrec = static_cast<const uint8_t*>(a.v_records);

    struct StepRef {
        int id, h;
        bool ok;
    };
    auto step_ref = [&](int k) {
        StepRef r;
        r.h = k % TS;
        r.id = k < nst ? a.block_table[(int64_t)bs * a.max_pages + sp + split + (k / TS) * a.nsplit] : -1;
        r.ok = k < nst && r.id >= 0 && (int64_t)r.id < a.n_qpages;
        return r;
    };

    uint32_t kw[NKP][PREK ? KW : 1];
    uint32_t vw[NS][PREV ? VHW : 1];
    uint32_t ksz = 0, vsz = 0;
    uint32_t ckr[NS][2], cvr[(NS + 1) / 2];  // fp16 column scales, two per word
#pragma unroll
    for (int c = 0; c < NKP; c++)
#pragma unroll
        for (int k = 0; k < (PREK ? KW : 1); k++) kw[c][k] = 0;
#pragma unroll
    for (int r = 0; r < NS; r++) {
        cvr[r >> 1] = 0;
        ckr[r][0] = ckr[r][1] = 0;
#pragma unroll
        for (int k = 0; k < (PREV ? VHW : 1); k++) vw[r][k] = 0;
    }
    auto issue_k = [&](const StepRef& r) {
        if (!r.ok) return;
        const uint8_t* rk = krec + ((int64_t)r.id * a.H + kvh) * KREC;
        const int tok = 64 * r.h + lane;
        if constexpr (PREK) {
#pragma unroll
            for (int c = 0; c < NKP; c++) load_words(kw[c], rk + (int64_t)tok * KROW + (NC * wave + c) * KCH, KW / 4);
        }
        ksz = reinterpret_cast<const uint32_t*>(rk + KCB)[tok];
        if (r.h == 0) {
            const uint16_t* ck = reinterpret_cast<const uint16_t*>(rk + KCB + 4 * T);
#pragma unroll
            for (int r2 = 0; r2 < NS; r2++) {
                const int i = 32 * (r2 >> 1) + blk + 16 * (r2 & 1) + (DH / 4) * wave;
                ckr[r2][0] = (uint32_t)ck[code_of<KB>(i, 0)] | ((uint32_t)ck[code_of<KB>(i, 1)] << 16);
                ckr[r2][1] = (uint32_t)ck[code_of<KB>(i, 2)] | ((uint32_t)ck[code_of<KB>(i, 3)] << 16);
            }
        }
    };
    auto issue_v = [&](const StepRef& r) {
        if (!r.ok) return;
        const uint8_t* rv = vrec + ((int64_t)r.id * a.H + kvh) * VREC;
#pragma unroll
        for (int sv = 0; sv < NS; sv++) {
            if constexpr (PREV) load_seg<VHW>(vw[sv], rv + vseg(r.h, 64 * (NS * wave + sv) + lane));
            if (r.h == 0) {
                const uint32_t c16 = reinterpret_cast<const uint16_t*>(rv + VCB + 4 * T)[64 * (NS * wave + sv) + lane];
                cvr[sv >> 1] = (sv & 1) ? (cvr[sv >> 1] | (c16 << 16)) : c16;
            }
        }
        vsz = reinterpret_cast<const uint32_t*>(rv + VCB)[64 * r.h + lane];
    };

    h4 qa[NS], qal[NS];  // score operands q' * C_K of the current page, high and low parts
    float sq[G];         // their sums per head
    float cvv[NS];       // value column scales of this lane's channels
#pragma unroll
    for (int g = 0; g < G; g++) sq[g] = 0.f;
#pragma unroll
    for (int r = 0; r < NS; r++) {
        qa[r] = qal[r] = h4{0, 0, 0, 0};
        cvv[r] = 0.f;
    }

    StepRef cur = step_ref(0);
    issue_k(cur);
    issue_v(cur);

    for (int k = 0; k < nst; k++) {
        const StepRef nxt = step_ref(k + 1);
        if (!cur.ok) {  // uniform: a page whose id is outside the record pool is skipped
            issue_k(nxt);
            issue_v(nxt);
            cur = nxt;
            continue;
        }
        const int id = cur.id;
        const int tok = 64 * cur.h + lane;
        const uint8_t* rk = krec + ((int64_t)id * a.H + kvh) * KREC;
        const uint8_t* rv = vrec + ((int64_t)id * a.H + kvh) * VREC;

        // ---- scores, lane = token ----
        float s[G];
        {
            if (cur.h == 0) {
                // score operands of the new page (fp16 high and low parts) and
                // their per-head sums, both from one fp32 product per channel
                // (the MFMA and the sum must see the same high part)
                float part = 0.f;
#pragma unroll
                for (int r = 0; r < NS; r++) {
#pragma unroll
                    for (int kk = 0; kk < 4; kk++) {
                        const float x =
                            fp32_value(qv[r][kk] * half_bits_to_float((ckr[r][kk >> 1] >> (16 * (kk & 1))) & 0xffffu));
                        const _Float16 hi = (_Float16)x;
                        const _Float16 lo = (_Float16)(x - (float)hi);
                        qa[r][kk] = hi;
                        qal[r][kk] = lo;
                        part += (float)hi + (float)lo;
                    }
                    cvv[r] = half_bits_to_float((cvr[r >> 1] >> (16 * (r & 1))) & 0xffffu);
                }
                part = sum_blocks_half(part);  // lanes g and 32 + g hold the halves' sums for head g
#pragma unroll
                for (int g = 0; g < G; g++)
                    sq[g] = i2f(__builtin_amdgcn_readlane(f2i(part), g)) + i2f(__builtin_amdgcn_readlane(f2i(part), 32 + g));
            }
            f4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < NC; c++) {
                uint32_t w[KW];
                if (PREK && c < NKP) {
#pragma unroll
                    for (int kk = 0; kk < KW; kk++) w[kk] = kw[c < NKP ? c : 0][PREK ? kk : 0];
                } else {
                    load_words(w, rk + (int64_t)tok * KROW + (NC * wave + c) * KCH, KW / 4);
                }
                static_for<32>([&](auto ic) {
                    constexpr int il = decltype(ic)::value;
                    const h4 bop = code_operand<KB>(w, il);
                    acc0 = mfma_bcast<il & 15>(qa[2 * c + (il >> 4)], bop, acc0);
                    acc1 = mfma_bcast<il & 15>(qal[2 * c + (il >> 4)], bop, acc1);
                });
            }
            const f4 R = acc0 + acc1;
            const float S = half_bits_to_float(ksz & 0xffffu), Z = half_bits_to_float(ksz >> 16);
            const float fs = FK * S, zc = Z - fs;
#pragma unroll
            for (int g = 0; g < G; g++) s[g] = sm2 * fmaf(fs, R[g], sq[g] * zc);
            if constexpr (NWV > 1) {
                // the score is linear in the channel halves: sum the waves'
                // partials (same order in every wave, so all see equal scores)
#pragma unroll
                for (int g = 0; g < G; g++) xs[k & 1][wave][g][lane] = s[g];
                __syncthreads();
#pragma unroll
                for (int g = 0; g < G; g++) {
                    float t = xs[k & 1][0][g][lane];
#pragma unroll
                    for (int w2 = 1; w2 < NWV; w2++) t += xs[k & 1][w2][g][lane];
                    s[g] = t;
                }
            }
        }
        issue_k(nxt);  // the key registers are free

        // ---- online softmax over the step (log2 domain) ----
        float p[G];
#pragma unroll
        for (int g = 0; g < G; g++) {
            const float mx = wave_max_all(s[g]);
            const float mnew = fmaxf(mrun[g], mx);  // finite: the step holds a valid token
            const float alpha = mrun[g] == -INFINITY ? 0.f : exp2f(mrun[g] - mnew);
            mrun[g] = mnew;
            lp[g] *= alpha;
#pragma unroll
            for (int sv = 0; sv < NS; sv++) accr[sv][g] *= alpha;
            p[g] = exp2f(s[g] - mnew);
            lp[g] += p[g];
        }

        {
            // weights times S_V (fp16 high and low parts) into LDS by operand
            // position; the constant 1 of the code operands returns through
            // sum (p Zp - 2^B p S).  Both parts come from one fp32 value, so
            // that e below subtracts exactly what the MFMA adds.  Each head's
            // weights are scaled by 2^(14 - e), e the exponent of its largest
            // weight of the step: the step's weights then stay in fp16's
            // normal range down to 2^-28 of that weight, where otherwise most
            // weights of a long sequence (far below the running maximum) would
            // be fp16 subnormals, whose treatment by the MFMA is not that of
            // the fp32 sum e.
            const float S = half_bits_to_float(vsz & 0xffffu), Z = half_bits_to_float(vsz >> 16);
            const int pos = pos_of<VB>(lane);
            float pmax[G], mxw[G], fvs[G], e[G];
#pragma unroll
            for (int g = 0; g < G; g++) pmax[g] = p[g] * S;
            wave_reduce4<true>(pmax, mxw);
#pragma unroll
            for (int g = 0; g < G; g++) {
                const int ex = frexp_exp(mxw[g]);
                const float x = fp32_value(__builtin_amdgcn_ldexpf(p[g] * S, 14 - ex));
                fvs[g] = __builtin_amdgcn_ldexpf(FV, ex - 14);
                const _Float16 hi = (_Float16)x;
                const _Float16 lo = (_Float16)(x - (float)hi);
                pt[wave][0][g][pos] = hi;
                pt[wave][1][g][pos] = lo;
                e[g] = fmaf(p[g], Z, -fvs[g] * ((float)hi + (float)lo));
            }
            float E[G];
#pragma unroll
            for (int g = 0; g < G; g++) E[g] = wave_sum_all(e[g]);
            wave_sync();
            const h4 pa = *reinterpret_cast<const h4*>(&pt[wave][0][m][4 * blk]);
            const h4 pal = *reinterpret_cast<const h4*>(&pt[wave][1][m][4 * blk]);
#pragma unroll
            for (int sv = 0; sv < NS; sv++) {
                uint32_t w[VHW];
                if constexpr (PREV) {
#pragma unroll
                    for (int kk = 0; kk < VHW; kk++) w[kk] = vw[sv][PREV ? kk : 0];
                } else {
                    load_seg<VHW>(w, rv + vseg(cur.h, 64 * (NS * wave + sv) + lane));
                }
                f4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
                static_for<16>([&](auto ic) {
                    constexpr int i = decltype(ic)::value;
                    const h4 bop = code_operand<VB>(w, i);
                    acc0 = mfma_bcast<i>(pa, bop, acc0);
                    acc1 = mfma_bcast<i>(pal, bop, acc1);
                });
                const f4 R = acc0 + acc1;
#pragma unroll
                for (int g = 0; g < G; g++) accr[sv][g] = fmaf(cvv[sv], fmaf(fvs[g], R[g], E[g]), accr[sv][g]);
            }
            wave_sync();  // pt is rewritten by the next step
        }
        issue_v(nxt);  // the value registers are free
        cur = nxt;
    }

    // ---- partial of this split: m, l, rotated-basis and fp16 value sums ----
    float* wsp = a.ws + (int64_t)a.B * Hq * D;
#pragma unroll
    for (int g = 0; g < G; g++) {
        const float lt = wave_sum_all(lp[g]);
        float* o = wsp + (((int64_t)b * Hq + h * G + g) * (a.nsplit + a.nfsplit) + split) * WS;
        if (lane == 0 && wave == 0) {
            o[0] = mrun[g];
            o[1] = lt;
        }
#pragma unroll
        for (int sv = 0; sv < NS; sv++) o[4 + 64 * (NS * wave + sv) + lane] = accr[sv][g];
    }
}

// ---- int8 operands -------------------------------------------------------------
typedef int i4v __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// 4 of 16 6-bit codes (bits 24 e .. 24 e + 23 of the 3 words w) as int8 bytes
template <int B>
__device__ __forceinline__ int code_bytes(const uint32_t* w, int e) {
    static_assert(B == 6, "6-bit codes only");
    // t: low half = bits 0..15 of the run, high half = bits 8..23
    uint32_t t;
    if (e == 0) t = __builtin_amdgcn_perm(w[0], w[0], 0x02010100u);
    else if (e == 1) t = __builtin_amdgcn_perm(w[1], w[0], 0x05040403u);
    else if (e == 2) t = __builtin_amdgcn_perm(w[2], w[1], 0x04030302u);
    else t = __builtin_amdgcn_perm(w[2], w[2], 0x03020201u);
    // low half: codes 0, 1 at bits 0-5, 6-11; high half >> 4: codes 2, 3 there
    const u16x2 hh = __builtin_bit_cast(u16x2, t) >> (u16x2){0, 4};
    const uint32_t uu = __builtin_bit_cast(uint32_t, hh);
    const uint32_t vv = __builtin_bit_cast(uint32_t, hh << (u16x2){2, 2});  // codes 1, 3 to bits 8-13
    return (int)((uu & 0x003F003Fu) | (vv & 0x3F003F00u));
}

// x (|x| < 2^21 after scaling) rounded to an integer X = d2 65536 + d1 256 + d0
// with balanced digits d in [-128, 127]: bytes 0, 1, 2 of the result are d0,
// d1, d2 as int8 (adding 0x808080 makes each digit byte d + 128; the xor
// turns that back into d's two's-complement byte).
__device__ __forceinline__ uint32_t digits3(float x) {
    const int X = (int)__builtin_rintf(x);
    return ((uint32_t)X + 0x808080u) ^ 0x808080u;
}

// z[L] = digit L of y0, y1, y2, y3 in bytes 0..3
__device__ __forceinline__ void digit_levels(uint32_t y0, uint32_t y1, uint32_t y2, uint32_t y3, int (&z)[3]) {
    const uint32_t a = __builtin_amdgcn_perm(y1, y0, 0x05010400u);  // y0.0 y1.0 y0.1 y1.1
    const uint32_t b = __builtin_amdgcn_perm(y3, y2, 0x05010400u);  // y2.0 y3.0 y2.1 y3.1
    z[0] = (int)__builtin_amdgcn_perm(b, a, 0x05040100u);
    z[1] = (int)__builtin_amdgcn_perm(b, a, 0x07060302u);
    z[2] = (int)(__builtin_amdgcn_perm(y1, y0, 0x0c0c0602u) | __builtin_amdgcn_perm(y3, y2, 0x06020c0cu));
}

// max and sum over the 16 lanes of one residue class mod 4
__device__ __forceinline__ float max_class4(float v) {
    v = fmaxf(v, i2f(__builtin_amdgcn_update_dpp(f2i(v), f2i(v), 0x124, 0xF, 0xF, false)));  // row_ror 4
    v = fmaxf(v, i2f(__builtin_amdgcn_update_dpp(f2i(v), f2i(v), 0x128, 0xF, 0xF, false)));  // row_ror 8
    const auto a16 = __builtin_amdgcn_permlane16_swap((unsigned)f2i(v), (unsigned)f2i(v), false, false);
    v = fmaxf(i2f((int)a16[0]), i2f((int)a16[1]));
    const auto a32 = __builtin_amdgcn_permlane32_swap((unsigned)f2i(v), (unsigned)f2i(v), false, false);
    return fmaxf(i2f((int)a32[0]), i2f((int)a32[1]));
}
__device__ __forceinline__ float sum_class4(float v) {
    v += i2f(__builtin_amdgcn_update_dpp(0, f2i(v), 0x124, 0xF, 0xF, true));  // row_ror 4
    v += i2f(__builtin_amdgcn_update_dpp(0, f2i(v), 0x128, 0xF, 0xF, true));  // row_ror 8
    const auto a16 = __builtin_amdgcn_permlane16_swap((unsigned)f2i(v), (unsigned)f2i(v), false, false);
    v = i2f((int)a16[0]) + i2f((int)a16[1]);
    const auto a32 = __builtin_amdgcn_permlane32_swap((unsigned)f2i(v), (unsigned)f2i(v), false, false);
    return i2f((int)a32[0]) + i2f((int)a32[1]);
}

// ---- D = 128: scores and value sums on the 32x32x32 int8 MFMA --------------
//
// One wave per (split, KV head, sequence), 64 tokens per step, as above, but
// each contraction is a handful of 32x32x32 int8 MFMAs (32 tokens or 32
// channels per instruction).  The rows of the int8 operand are (digit level
// L, query head g) = 4 L + g, 12 of 32 used: the query times C of a page (or
// the softmax weights times S of a step) is scaled by a power of two below
// 2^21, rounded to an integer and split into three balanced base-256 digits,
// so the int32 results are exact and recombine in fp32.  The codes are the
// other operand, one byte per code.
//
// Lane l of a 32x32 result holds rows {8 j + 4 (l >> 5) + i}, i.e. levels 0
// and 2 in the lower half-wave and level 1 in the upper one, for column
// l & 31.  Two results (token blocks 0/1, or channel blocks 2 s / 2 s + 1)
// are paired with v_permlane32_swap so that every lane ends with all three
// levels of its own column: lane l holds token l of the step (scores) or
// channel 64 s + l (value sums).
typedef int i16v __attribute__((ext_vector_type(16)));

// 16 codes (B bits each, LSB-first words w[0 .. B/2-1]) as 16 int8 bytes;
// byte j holds code perm16<B>(j)
template <int B>
__device__ __forceinline__ i4v codes16(const uint32_t* w) {
    if constexpr (B == 4) {
        return i4v{(int)(w[0] & 0x0F0F0F0Fu), (int)((w[0] >> 4) & 0x0F0F0F0Fu), (int)(w[1] & 0x0F0F0F0Fu),
                   (int)((w[1] >> 4) & 0x0F0F0F0Fu)};
    } else if constexpr (B == 2) {
        return i4v{(int)(w[0] & 0x03030303u), (int)((w[0] >> 2) & 0x03030303u), (int)((w[0] >> 4) & 0x03030303u),
                   (int)((w[0] >> 6) & 0x03030303u)};
    } else {
        return i4v{code_bytes<6>(w, 0), code_bytes<6>(w, 1), code_bytes<6>(w, 2), code_bytes<6>(w, 3)};
    }
}
// element of the 16 held in byte j by codes16<B>, and its inverse
template <int B>
__host__ __device__ constexpr int perm16(int j) {
    if constexpr (B == 4) return (j & 8) + 2 * (j & 3) + ((j >> 2) & 1);
    else if constexpr (B == 2) return 4 * (j & 3) + (j >> 2);
    else return j;
}
template <int B>
__host__ __device__ constexpr int perm16_inv(int c) {
    if constexpr (B == 4) return (c & 8) + 4 * (c & 1) + ((c >> 1) & 3);
    else if constexpr (B == 2) return 4 * (c & 3) + (c >> 2);
    else return c;
}

__device__ __forceinline__ i16v mfma32_i8(i4v a, i4v b, i16v c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

// x: lanes 0-31 hold column c0's L0 at x[g] and L2 at x[4 + g], lanes 32-63
// its L1 at x[g]; y likewise for column c1.  Returns, per lane, 65536 L2 +
// 256 L1 + L0 of its own column (c0 in the lower half, c1 in the upper half)
// for g = 0..3; L0 + 256 L1 is summed in int32 (each level is a sum of at
// most 128 digit-code products, below 2^21 in magnitude).
__device__ __forceinline__ f4 pair_levels(const i16v& x, const i16v& y) {
    f4 r;
#pragma unroll
    for (int g = 0; g < 4; g++) {
        const auto s01 = __builtin_amdgcn_permlane32_swap((unsigned)x[g], (unsigned)y[g], false, false);
        const auto s2 = __builtin_amdgcn_permlane32_swap((unsigned)x[4 + g], (unsigned)y[4 + g], false, false);
        // s01[0]: L0 of the lane's column, s01[1]: L1; s2[0]: L2
        r[g] = fmaf((float)(int)s2[0], 65536.0f, (float)((int)s01[0] + (int)(s01[1] << 8)));
    }
    return r;
}

template <int T, int KB, int VB>
__global__ void __launch_bounds__(64) decode_split128_kernel(DecodeArgs a) {
    constexpr int D = 128, G = 4;
    constexpr int TS = T / 64;            // 64-token steps of a page
    constexpr int KCB = T * D * KB / 8;
    constexpr int VCB = T * D * VB / 8;
    constexpr int KREC = KCB + 4 * T + 2 * D;
    constexpr int VREC = VCB + 4 * T + 2 * D;
    constexpr int KROW = D * KB / 8;      // code bytes of a token
    constexpr int KW = KROW / 8;          // words of half a token row (64 channels)
    constexpr int VW = VB;                // words of 32 tokens of a channel
    constexpr int WS = D + 4;           // partial: m, l, pad, pad, value sums
    constexpr int QROW = D, WROW = 64;    // bytes per row of the query / weight digit tables
    static_assert(KW == KB * 2 && (KROW / 2) % 16 == 0, "half token rows in 16-byte loads");

    // The LDS stage of one step, filled by LDS-DMA loads issued one step
    // ahead: key codes (the step's 64 token rows, 16-byte pieces swizzled for
    // KB = 4), the scale blocks of the page's K and V records (token scales
    // and column scales, loaded with the page's first step), value codes
    // (channel-major, the 8 VB bytes of a channel's 64 tokens).  fp16 slots
    // use the same memory for their weights.
    constexpr int KST = 64 * KROW;
    constexpr int VST = 128 * 8 * VB;
    constexpr int SB = 4 * T + 2 * D;     // scale block of a record
    constexpr int KSC = KST, VSC = KSC + SB, VSO = VSC + SB;
    constexpr int STAGE = VSO + VST;
    static_assert(SB % 16 == 0 && SB / 16 <= 64, "scale block in one 16-byte load");
    static_assert(STAGE >= 16 * 64 && KST % 1024 == 0 && VST % 1024 == 0, "stage sizes");
    __shared__ __attribute__((aligned(16))) uint8_t stage[STAGE];
    // digit tables, rows 4 L + g; row 12 stays zero (the unused operand rows)
    __shared__ __attribute__((aligned(16))) uint8_t qt[13 * QROW];
    __shared__ __attribute__((aligned(16))) uint8_t wt[13 * WROW];

    // grid z < B: quantized-page splits; z >= B: fp16 page slots, dispatched
    // after every split so that they fill the splits' tail
    if ((int)blockIdx.z >= a.B) {
        if ((int)blockIdx.x < a.nfsplit)
            fp16_block<D, T>(a, blockIdx.x, blockIdx.y, blockIdx.z - a.B, reinterpret_cast<float4*>(stage));
        return;
    }
    if ((int)blockIdx.x >= a.nsplit) return;
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x;
    const int half = lane >> 5, col = lane & 31;
    const int orow = min(col, 12);        // operand row of this lane (12: zeros)
    const int Hq = a.Hq;
    const float sm2 = a.sm_scale * kLog2e;

    if (lane < 32) reinterpret_cast<uint32_t*>(qt + 12 * QROW)[lane] = 0u;
    if (lane < 16) reinterpret_cast<uint32_t*>(wt + 12 * WROW)[lane] = 0u;

    // query digit builder: lane = (head g = lane & 3, q = lane >> 2) owns the
    // table positions 16 (q >> 1) + 4 u + k, u = 2 (q & 1) + i (i = 0, 1),
    // i.e. channels 16 (q >> 1) + perm16<KB>(4 u + k)
    const int bg = lane & 3, bq = lane >> 2;
    auto bchan = [&](int i, int k) { return 16 * (bq >> 1) + perm16<KB>(4 * (2 * (bq & 1) + i) + k); };
    // q' = H q / sqrt(D) of the wave's 4 heads, rotated here: lane (g = lane
    // >> 4, m = lane & 15) holds channels 8 m .. 8 m + 7 of head h G + g;
    // channel bits 0-2 are butterflies in registers, bits 3-6 (lane bits 0-3)
    // across lanes; the result goes through the (still idle) LDS stage to the
    // builder lanes.
    float qv[2][4];
    {
        const int g = lane >> 4, m = lane & 15;
        const int64_t qrow = ((int64_t)b * Hq + h * G + g) * D + 8 * m;
        float x[8];
        q_load<8>(a.q, a.q_dtype, qrow, x);
#pragma unroll
        for (int hs = 1; hs < 8; hs <<= 1)
#pragma unroll
            for (int e = 0; e < 8; e++)
                if ((e & hs) == 0) {
                    const float u = x[e], v = x[e + hs];
                    x[e] = u + v;
                    x[e + hs] = u - v;
                }
        // lane bit k: the lane with the bit set keeps partner - self, the other self + partner
        auto xstage = [&](auto bitc) {
            constexpr int BIT = decltype(bitc)::value;
            const float sg = ((lane >> BIT) & 1) ? -1.f : 1.f;
#pragma unroll
            for (int e = 0; e < 8; e++) x[e] = fmaf(sg, x[e], xor_lane<BIT>(x[e]));
        };
        xstage(std::integral_constant<int, 0>{});
        xstage(std::integral_constant<int, 1>{});
        xstage(std::integral_constant<int, 2>{});
        xstage(std::integral_constant<int, 3>{});
        float* qs = reinterpret_cast<float*>(stage);  // [4 heads][D]
        const float rs = 1.0f / sqrtf((float)D);
        *reinterpret_cast<float4*>(qs + g * D + 8 * m) = make_float4(x[0] * rs, x[1] * rs, x[2] * rs, x[3] * rs);
        *reinterpret_cast<float4*>(qs + g * D + 8 * m + 4) = make_float4(x[4] * rs, x[5] * rs, x[6] * rs, x[7] * rs);
        wave_sync();
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int k = 0; k < 4; k++) qv[i][k] = qs[bg * D + bchan(i, k)];
        wave_sync();  // the stage is reused by the loads below
    }

    // sequence length and page ids are wave-uniform (SGPRs)
    const int bs = b / a.M;  // sequence of query row b (its quantized pages lie before every query token)
    const int L = __builtin_amdgcn_readfirstlane(min(a.seq_lens[bs], a.max_pages * T));
    const int nq = (L - a.sink - a.tail >= T) ? (L - a.sink - a.tail) / T : 0;
    const int sp = a.sink / T;

    float mrun[G], lp[G], accr[2][G];
#pragma unroll
    for (int g = 0; g < G; g++) {
        mrun[g] = -INFINITY;
        lp[g] = 0.f;
        accr[0][g] = accr[1][g] = 0.f;
    }

    const int npg = __builtin_amdgcn_readfirstlane(nq > split ? (nq - split + a.nsplit - 1) / a.nsplit : 0);  // quantized pages of this split
    const int nst = npg * TS;
    const uint8_t* const krec = static_cast<const uint8_t*>(a.k_records);
    const uint8_t* const vrec = static_cast<const uint8_t*>(a.v_records);

    // the split's page ids, 64 at a time, page 64 c + l in lane l
    const int* const btrow = a.block_table + (int64_t)bs * a.max_pages + sp + split;
    auto page_ids = [&](int c) {
        const int i = 64 * c + lane;
        const int id = i < npg ? btrow[(int64_t)i * a.nsplit] : -1;
        asm volatile("" ::"v"(id));  // the load completes here, before any LDS-DMA load is in flight
        return id;
    };
    int ids = page_ids(0);
    struct StepRef {
        int id, h;
        bool ok;
    };
    auto step_ref = [&](int k) {
        StepRef r;
        r.h = k % TS;
        r.id = k < nst ? __builtin_amdgcn_readlane(ids, (k / TS) & 63) : -1;
        r.ok = k < nst && r.id >= 0 && (int64_t)r.id < a.n_qpages;
        return r;
    };

    // A step's operands in registers: the lane's half rows of tokens col and
    // 32 + col, the 32-token share of channels 32 cb + col (cb = 0..3), the
    // scale words of token `lane`, and on a page's first step the builder's 8
    // column scales of K and this lane's 2 of V.
    struct Buf {
        uint32_t kw[2][KW];
        uint32_t vw[4][VW];
        uint32_t ksz, vsz;
        uint32_t ck[4];   // fp16 pairs: C_K at bchan(i, 2 j), bchan(i, 2 j + 1), word 2 i + j
        uint32_t cv;      // fp16 pair: C_V of channels lane, 64 + lane
    };
    // Loads go through one buffer resource per pool (the pool sizes are below
    // 4 GiB, checked on the host): the record offset is a scalar offset, the
    // lane's part a 32-bit vector offset.
    const i4v rsk = raw_buffer(krec, (uint32_t)(a.n_qpages * a.H * KREC));
    const i4v rsv = raw_buffer(vrec, (uint32_t)(a.n_qpages * a.H * VREC));
    // key piece u (16 bytes; u = KB t + p for token t of the step) sits at
    // stage piece kswz(u): for KB = 2 and 4 the KB pieces of a row rotate
    // with bits 2-3 (KB = 4) or bit 3 (KB = 2) of the token, so that the 16
    // lanes of a 128-bit read pass (one piece of 16 consecutive tokens) hit 16
    // different 4-bank groups of the 64-bank LDS (kswz is an involution)
    auto kswz = [](int u) { return (KB == 4 || KB == 2) ? (u ^ ((u >> 4) & (KB - 1))) : u; };
    const uint32_t sb = lds_address(stage);
    // all of a step's loads into the stage
    auto issue = [&](const StepRef& r) {
        if (!r.ok) return;
        const uint32_t rec = (uint32_t)r.id * (uint32_t)a.H + (uint32_t)(h / a.GS);
        // byte offsets in the pools (each below 4 GiB) as unsigned 32-bit
        // values: the buffer load adds its scalar offset modulo 2^32
        const uint32_t sk = (uint32_t)__builtin_amdgcn_readfirstlane((int)(rec * (uint32_t)KREC));
        const uint32_t sv = (uint32_t)__builtin_amdgcn_readfirstlane((int)(rec * (uint32_t)VREC));
        // kswz(64 i + lane) = 64 i + kswz(lane): the KST / 1024 key loads
        // are runs under one M0 each
        static_assert(KST % 1024 == 0, "key runs");
        lds_dma16_runs<KST / 1024>(sb, rsk, 16 * kswz(lane), (int)(sk + (uint32_t)(KST * r.h)));
        if (r.h == 0 && lane < SB / 16) {  // the page's scale blocks
            lds_dma16(sb + KSC, rsk, 16 * lane, (int)(sk + (uint32_t)KCB));
            lds_dma16(sb + VSC, rsv, 16 * lane, (int)(sv + (uint32_t)VCB));
        }
        // piece u = channel u / (VB / 2), part u % (VB / 2): values are kept
        // in 64-token blocks, so a step's pieces are one contiguous run
        static_assert(VST % 1024 == 0, "value runs");
        lds_dma16_runs<VST / 1024>(sb + VSO, rsv, 16 * lane, (int)(sv + (uint32_t)((64 * D * VB / 8) * r.h)));
    };
    // the lane's operands of a step out of the stage (after its loads have
    // landed); once these reads are done the stage may be refilled
    auto fetch = [&](const StepRef& r, Buf& f) {
#pragma unroll
        for (int tb = 0; tb < 2; tb++)
#pragma unroll
            for (int j = 0; j < KB / 2; j++) {
                const int u = KB * (32 * tb + col) + (KB / 2) * half + j;
                const uint4 v = *reinterpret_cast<const uint4*>(stage + 16 * kswz(u));
                f.kw[tb][4 * j] = v.x; f.kw[tb][4 * j + 1] = v.y; f.kw[tb][4 * j + 2] = v.z; f.kw[tb][4 * j + 3] = v.w;
            }
#pragma unroll
        for (int cb = 0; cb < 4; cb++)
#pragma unroll
            for (int j = 0; j < VW / 2; j++) {
                const uint2 v = *reinterpret_cast<const uint2*>(stage + VSO + (32 * cb + col) * 8 * VB + 4 * VB * half + 8 * j);
                f.vw[cb][2 * j] = v.x; f.vw[cb][2 * j + 1] = v.y;
            }
        f.ksz = *reinterpret_cast<const uint32_t*>(stage + KSC + 4 * (64 * r.h + lane));
        f.vsz = *reinterpret_cast<const uint32_t*>(stage + VSC + 4 * (64 * r.h + lane));
        if (r.h == 0) {
            const uint16_t* ckc = reinterpret_cast<const uint16_t*>(stage + KSC + 4 * T);
            const uint16_t* cvc = reinterpret_cast<const uint16_t*>(stage + VSC + 4 * T);
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < 2; j++)
                    f.ck[2 * i + j] = (uint32_t)ckc[bchan(i, 2 * j)] | ((uint32_t)ckc[bchan(i, 2 * j + 1)] << 16);
            f.cv = (uint32_t)cvc[lane] | ((uint32_t)cvc[64 + lane] << 16);
        }
    };

    float qs[G], sqs[G];  // per head: sm2 * 2^(e - 21) and sm2 * sum(q' * C) of the current page
    float cvv[2];         // value column scales of channels lane, 64 + lane
#pragma unroll
    for (int g = 0; g < G; g++) qs[g] = sqs[g] = 0.f;
    cvv[0] = cvv[1] = 0.f;
    const int wpos = 16 * (lane >> 4) + perm16_inv<VB>(lane & 15);  // weight-table position of token `lane`

    auto step = [&](const StepRef& cur, const StepRef& nxt, Buf& u) {
        if (!cur.ok) {  // uniform: a page whose id is outside the record pool is skipped
            issue(nxt);
            return;
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");    // this step's stage has landed
        fetch(cur, u);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // ... and has been read
        issue(nxt);
        if (cur.h == 0) {
            // query digits of the new page into the table: q~ = q' * C_K, per
            // head scaled so that max |q~| 2^(21 - e) < 2^21
            float qt4[2][4];
            float mx = 0.f, sum = 0.f;
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int k = 0; k < 4; k++) {
                    const uint32_t w = u.ck[2 * i + (k >> 1)];
                    qt4[i][k] = qv[i][k] * half_bits_to_float((w >> (16 * (k & 1))) & 0xffffu);
                    mx = fmaxf(mx, fabsf(qt4[i][k]));
                    sum += qt4[i][k];
                }
            mx = max_class4(mx);    // the 16 lanes of head bg
            sum = sum_class4(sum);
            const int e = frexp_exp(mx);
#pragma unroll
            for (int i = 0; i < 2; i++) {
                uint32_t y[4];
#pragma unroll
                for (int k = 0; k < 4; k++) y[k] = digits3(__builtin_amdgcn_ldexpf(qt4[i][k], 21 - e));
                int z[3];
                digit_levels(y[0], y[1], y[2], y[3], z);
                const int pos = 16 * (bq >> 1) + 4 * (2 * (bq & 1) + i);
#pragma unroll
                for (int lv = 0; lv < 3; lv++) *reinterpret_cast<int*>(qt + (4 * lv + bg) * QROW + pos) = z[lv];
            }
            const float qsl = __builtin_amdgcn_ldexpf(sm2, e - 21);
            const float sql = sm2 * sum;
#pragma unroll
            for (int g = 0; g < G; g++) {  // lanes 0..3 hold heads 0..3
                qs[g] = i2f(__builtin_amdgcn_readlane(f2i(qsl), g));
                sqs[g] = i2f(__builtin_amdgcn_readlane(f2i(sql), g));
            }
            cvv[0] = half_bits_to_float(u.cv & 0xffffu);
            cvv[1] = half_bits_to_float(u.cv >> 16);
            wave_sync();
        }

        // ---- scores: token blocks 0 and 1, k-step ks covers channels
        // 64 half + 16 ks + perm16(j) in byte j of both operands ----
        float s[G];
        {
            i16v d0 = {}, d1 = {};
#pragma unroll
            for (int ks = 0; ks < 4; ks++) {
                const i4v aq = *reinterpret_cast<const i4v*>(qt + orow * QROW + 16 * (4 * half + ks));
                d0 = mfma32_i8(aq, codes16<KB>(&u.kw[0][ks * KB / 2]), d0);
                d1 = mfma32_i8(aq, codes16<KB>(&u.kw[1][ks * KB / 2]), d1);
            }
            const f4 R = pair_levels(d0, d1);  // token `lane`
            const float S = half_bits_to_float(u.ksz & 0xffffu), Z = half_bits_to_float(u.ksz >> 16);
#pragma unroll
            for (int g = 0; g < G; g++) s[g] = fmaf(S * qs[g], R[g], Z * sqs[g]);
        }

        // ---- online softmax over the step (log2 domain) ----
        float p[G];
        {
            float mx[G], t[G] = {s[0], s[1], s[2], s[3]};
            wave_reduce4<true>(t, mx);
#pragma unroll
            for (int g = 0; g < G; g++) {
                const float mnew = fmaxf(mrun[g], mx[g]);  // finite: the step holds a valid token
                const float alpha = mrun[g] == -INFINITY ? 0.f : exp2f(mrun[g] - mnew);
                mrun[g] = mnew;
                lp[g] *= alpha;
                accr[0][g] *= alpha;
                accr[1][g] *= alpha;
                p[g] = exp2f(s[g] - mnew);
                lp[g] += p[g];
            }
        }

        // ---- value sums: weights p S_V as digit levels through the table;
        // k-step ks covers tokens 32 half + 16 ks + perm16(j) ----
        {
            const float S = half_bits_to_float(u.vsz & 0xffffu), Z = half_bits_to_float(u.vsz >> 16);
            // each head's weights p S_V scaled by 2^(21 - e), e the exponent of
            // that head's largest weight of the step: every step keeps 21 bits
            // relative to its own largest contribution (a step whose tokens all
            // score far below the running maximum would otherwise keep only a
            // few bits, and their rounding -- times non-negative codes -- would
            // not cancel against the zero-point sum)
            float ps[G], pmax[G], E[G], pz[G];
#pragma unroll
            for (int g = 0; g < G; g++) ps[g] = pmax[g] = p[g] * S;
            float mxw[G];
            wave_reduce4<true>(pmax, mxw);
            float wsc[G];
#pragma unroll
            for (int g = 0; g < G; g++) {
                const int e = frexp_exp(mxw[g]);
                wsc[g] = __builtin_amdgcn_ldexpf(1.0f, e - 21);
                const uint32_t y = digits3(__builtin_amdgcn_ldexpf(ps[g], 21 - e));
                wt[(0 + g) * WROW + wpos] = (uint8_t)y;
                wt[(4 + g) * WROW + wpos] = (uint8_t)(y >> 8);
                wt[(8 + g) * WROW + wpos] = (uint8_t)(y >> 16);
                pz[g] = p[g] * Z;
            }
            wave_reduce4<false>(pz, E);
            wave_sync();
            const i4v aw0 = *reinterpret_cast<const i4v*>(wt + orow * WROW + 16 * (2 * half + 0));
            const i4v aw1 = *reinterpret_cast<const i4v*>(wt + orow * WROW + 16 * (2 * half + 1));
#pragma unroll
            for (int sv = 0; sv < 2; sv++) {
                i16v d0 = {}, d1 = {};
                d0 = mfma32_i8(aw0, codes16<VB>(&u.vw[2 * sv][0]), d0);
                d1 = mfma32_i8(aw0, codes16<VB>(&u.vw[2 * sv + 1][0]), d1);
                d0 = mfma32_i8(aw1, codes16<VB>(&u.vw[2 * sv][VB / 2]), d0);
                d1 = mfma32_i8(aw1, codes16<VB>(&u.vw[2 * sv + 1][VB / 2]), d1);
                const f4 R = pair_levels(d0, d1);  // channel 64 sv + lane
#pragma unroll
                for (int g = 0; g < G; g++) accr[sv][g] = fmaf(cvv[sv], fmaf(wsc[g], R[g], E[g]), accr[sv][g]);
            }
            wave_sync();  // the tables are rewritten by later steps
        }
    };

    Buf buf;
    StepRef cur = step_ref(0);
    issue(cur);
    for (int k = 0; k < nst; k++) {
        if ((k + 1) % (64 * TS) == 0 && k + 1 < nst) {  // the next 64 pages' ids (the stage's loads wait)
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            ids = page_ids((k + 1) / (64 * TS));
        }
        const StepRef nx = step_ref(k + 1);
        step(cur, nx, buf);
        cur = nx;
    }

    // ---- partial of this split: m, l, rotated-basis and fp16 value sums ----
    float* wsp = a.ws + (int64_t)a.B * Hq * D;
#pragma unroll
    for (int g = 0; g < G; g++) {
        const float lt = wave_sum_all(lp[g]);
        float* o = wsp + (((int64_t)b * Hq + h * G + g) * (a.nsplit + a.nfsplit) + split) * WS;
        if (lane == 0) {
            o[0] = mrun[g];
            o[1] = lt;
        }
        o[4 + lane] = accr[0][g];
        o[4 + 64 + lane] = accr[1][g];
    }
}

// q' = H q / sqrt(D) in fp32, one workgroup of D/2 threads per (sequence, query head)
template <int D>
__global__ void __launch_bounds__(D / 2) qrot_kernel(const void* __restrict__ q, int q_dtype, float* __restrict__ qr) {
    __shared__ float x[D];
    const int bh = blockIdx.x, k = threadIdx.x;
    for (int j = k; j < D; j += D / 2) x[j] = q_at(q, q_dtype, (int64_t)bh * D + j);
    __syncthreads();
    for (int hs = 1; hs < D; hs <<= 1) {
        const int i0 = (k / hs) * 2 * hs + (k % hs), i1 = i0 + hs;
        const float u = x[i0], v = x[i1];
        __syncthreads();
        x[i0] = u + v;
        x[i1] = u - v;
        __syncthreads();
    }
    const float rs = 1.0f / sqrtf((float)D);
    for (int j = k; j < D; j += D / 2) qr[(int64_t)bh * D + j] = x[j] * rs;
}

template <int D>
hipError_t launch_combine(const DecodeArgs& a, hipStream_t st) {
    return launch_split_merge<D>(a.ws + (int64_t)a.B * a.Hq * D, a.out, a.B * a.Hq, a.nsplit, a.nsplit + a.nfsplit, st);
}

// Grid x of a split launch.  With several query rows per sequence (M > 1)
// the rows of one sequence are adjacent in grid z; x is padded (the extra
// workgroups return at once) so that x * y is a multiple of 8, which puts
// the rows' workgroups -- dispatched to the 8 XCDs in turn by linear id -- on
// one XCD, where they read the sequence's records through one L2.
inline unsigned split_grid_x(unsigned gx, unsigned gy, int M, int GS) {
    if (GS > 1)  // the query-head groups of one KV head are adjacent in y
        while (gx % 8u) gx++;
    else if (M > 1)
        while ((gx * gy) % 8u) gx++;
    return gx;
}

template <int D, int T, int KB, int VB>
hipError_t launch_gqa(const DecodeArgs& a, hipStream_t st) {
    hipError_t e;
    if constexpr (D != 128) {  // the head_dim 128 split kernel rotates its queries itself
        hipLaunchKernelGGL((qrot_kernel<D>), dim3(a.B * a.Hq), dim3(D / 2), 0, st, a.q, a.q_dtype, a.ws);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // one launch: the quantized-page splits (z < B), then the fp16 page slots
    constexpr int NWV = D == 128 ? 1 : split_waves<D>();
    const int nfx = (a.nfsplit + NWV - 1) / NWV;  // fp16 slots: one per wave
    const int gy = a.H * a.GS;
    const dim3 grid(split_grid_x(a.nsplit > nfx ? a.nsplit : nfx, gy, a.M, a.GS), gy, a.nfsplit > 0 ? 2 * a.B : a.B);
    if constexpr (D == 128)
        hipLaunchKernelGGL((decode_split128_kernel<T, KB, VB>), grid, dim3(64), 0, st, a);
    else
        hipLaunchKernelGGL((decode_split_kernel<D, T, KB, VB>), grid, dim3(64 * NWV), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_combine<D>(a, st);
}

}  // namespace

}  // namespace kvarn
