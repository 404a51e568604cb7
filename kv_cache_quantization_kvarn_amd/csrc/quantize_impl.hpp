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

// lane bit carrying channel-group bit k
__device__ __forceinline__ constexpr int cg_lane_bit(int k) {
    return k == 0 ? 0 : k == 1 ? 1 : k == 2 ? 3 : k == 3 ? 2 : 4;
}

template <int BIT>
__device__ __forceinline__ float butterfly(float v, int lane) {
    // lower lane (bit clear): v + partner; upper lane: partner - v
    const float p = xor_lane<BIT>(v);
    return ((lane >> BIT) & 1) ? (p - v) : (v + p);
}

template <int CGB>
__device__ __forceinline__ float row_sum(float v) {
    v += xor_lane<0>(v);
    v += xor_lane<1>(v);
    v += xor_lane<3>(v);
    if constexpr (CGB >= 4) v += xor_lane<2>(v);
    if constexpr (CGB >= 5) v += xor_lane<4>(v);
    return v;
}

template <int CGB>
__device__ __forceinline__ float row_min(float v) {
    v = fminf(v, xor_lane<0>(v));
    v = fminf(v, xor_lane<1>(v));
    v = fminf(v, xor_lane<3>(v));
    if constexpr (CGB >= 4) v = fminf(v, xor_lane<2>(v));
    if constexpr (CGB >= 5) v = fminf(v, xor_lane<4>(v));
    return v;
}

template <int CGB>
__device__ __forceinline__ float row_max(float v) {
    v = fmaxf(v, xor_lane<0>(v));
    v = fmaxf(v, xor_lane<1>(v));
    v = fmaxf(v, xor_lane<3>(v));
    if constexpr (CGB >= 4) v = fmaxf(v, xor_lane<2>(v));
    if constexpr (CGB >= 5) v = fmaxf(v, xor_lane<4>(v));
    return v;
}

__device__ __forceinline__ bool usable(float s) { return s > 0.f && s <= 3.0e38f; }

template <int D, int T>
struct TileShape {
    static constexpr int LPR = D / QC;                        // lanes per token row
    static constexpr int CGB = LPR == 8 ? 3 : LPR == 16 ? 4 : 5;
    static constexpr int RGB = 6 - CGB;                       // row-group bits inside a wave
    static constexpr int RPW = QR << RGB;                     // rows per wave
    static constexpr int NW = T / RPW;                        // waves per workgroup
    static constexpr int NT = NW * 64;
    static constexpr int NSUB = (RGB == 3) ? 2 : 1;           // lane bit 2 left after the swaps
    static constexpr int SMEM_CODES = T * D;
    static constexpr int SMEM_PART = NW * NSUB * D * 4;
    static constexpr int SMEM = SMEM_CODES > SMEM_PART ? SMEM_CODES : SMEM_PART;
};

// One tile -> one record.  smem: TileShape::SMEM bytes; bvec: D floats.
template <int D, int T, int BITS, bool CHMAJOR>
__device__ __forceinline__ void quantize_tile(const uint16_t* __restrict__ tile, uint8_t* __restrict__ rec,
                                              uint8_t* smem, float* bvec, int32_t n_iters) {
    using S = TileShape<D, T>;
    constexpr int CGB = S::CGB, RGB = S::RGB, RPW = S::RPW, NW = S::NW, NT = S::NT, NSUB = S::NSUB;
    constexpr int QMAX = (1 << BITS) - 1;
    constexpr int CODE_BYTES = T * D * BITS / 8;
    constexpr int REC = CODE_BYTES + 4 * T + 2 * D;
    constexpr int NPART = (RGB >= 2) ? 4 : 8;          // column partials per lane after swaps
    constexpr bool KEEP_Y = D <= 256;                  // D = 512 rebuilds y from y^2 and signs
    static_assert(T * D / 64 == NT, "one lane per 64 values");
    static_assert(REC % 16 == 0, "records stay 16-byte aligned");

    float* colpart = reinterpret_cast<float*>(smem);

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

    // ---- stage 1: load the fp16 tile ---------------------------------------
    float y[QR][QC];
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
#pragma unroll
        for (int c = 0; c < QC; c++) {
            float v = y[r][c];
            v = butterfly<0>(v, lane);
            v = butterfly<1>(v, lane);
            v = butterfly<3>(v, lane);
            if constexpr (CGB >= 4) v = butterfly<2>(v, lane);
            if constexpr (CGB >= 5) v = butterfly<4>(v, lane);
            y[r][c] = v;
        }
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
            if (usable(s)) bvec[tid] = (float)T / s;
        }
        __syncthreads();
#pragma unroll
        for (int c4 = 0; c4 < QC / 4; c4++) {
            float4 v = *reinterpret_cast<const float4*>(bvec + ch0 + 4 * c4);
            bw[4 * c4 + 0] = v.x;
            bw[4 * c4 + 1] = v.y;
            bw[4 * c4 + 2] = v.z;
            bw[4 * c4 + 3] = v.w;
        }
        if (it == n_iters - 1) break;
        // row step
#pragma unroll
        for (int r = 0; r < QR; r++) {
            float s = A[r][0] * bw[0];
#pragma unroll
            for (int c = 1; c < QC; c++) s = fmaf(A[r][c], bw[c], s);
            s = row_sum<CGB>(s);
            if (usable(s)) aw[r] = (float)D / s;
        }
    }

    // ---- stage 4: per-token asymmetric round-to-nearest --------------------
    float ic[QC];
#pragma unroll
    for (int c = 0; c < QC; c++) ic[c] = sqrtf(bw[c]);  // 1 / c_j (unnormalized basis)
    uint32_t sz[QR];
    uint8_t* codes = smem;  // [record element order], one byte per code
    uint32_t cw[QR][QC / 4];
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
        mn = row_min<CGB>(mn);
        mx = row_max<CGB>(mx);
        const float range = mx - mn;
        const float s = range / (float)QMAX;
        const float inv = range > 0.f ? (float)QMAX / range : 0.f;
        sz[r] = float_to_half_bits(s) | (float_to_half_bits(mn) << 16);
#pragma unroll
        for (int c4 = 0; c4 < QC / 4; c4++) {
            uint32_t word = 0;
#pragma unroll
            for (int k = 0; k < 4; k++) {
                float u = (W[4 * c4 + k] - mn) * inv;
                float qf = fminf(fmaxf(rintf(u), 0.f), (float)QMAX);
                word |= (uint32_t)qf << (8 * k);
            }
            cw[r][c4] = word;
        }
    }
    // all statistics reads of the shared buffer are behind the last barrier;
    // the code bytes reuse it
    if constexpr (!CHMAJOR) {
#pragma unroll
        for (int r = 0; r < QR; r++) {
            uint4 v = make_uint4(cw[r][0], cw[r][1], cw[r][2], cw[r][3]);
            *reinterpret_cast<uint4*>(codes + (row0 + r) * D + ch0) = v;
        }
    } else {
#pragma unroll
        for (int c = 0; c < QC; c++) {
            uint32_t v = 0;
#pragma unroll
            for (int r = 0; r < QR; r++) v |= ((cw[r][c >> 2] >> (8 * (c & 3))) & 0xffu) << (8 * r);
            *reinterpret_cast<uint32_t*>(codes + (ch0 + c) * T + row0) = v;
        }
    }
    // per-token scale and zero-point: 4 consecutive tokens = 16 bytes
    if (cg == 0) {
        *reinterpret_cast<uint4*>(rec + CODE_BYTES + 4 * row0) = make_uint4(sz[0], sz[1], sz[2], sz[3]);
    }
    // column scales, normalized basis: C_j = 1 / sqrt(D * b_j)
    if (tid < D / 8) {
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; k++) {
            float c0 = 1.0f / sqrtf((float)D * bvec[8 * tid + 2 * k]);
            float c1 = 1.0f / sqrtf((float)D * bvec[8 * tid + 2 * k + 1]);
            w[k] = float_to_half_bits(c0) | (float_to_half_bits(c1) << 16);
        }
        *reinterpret_cast<uint4*>(rec + CODE_BYTES + 4 * T + 16 * tid) = make_uint4(w[0], w[1], w[2], w[3]);
    }
    __syncthreads();

    // ---- stage 5: pack 64 codes per thread, LSB first -----------------------
    {
        const uint4* cp = reinterpret_cast<const uint4*>(codes + 64 * tid);
        uint32_t in[16];
#pragma unroll
        for (int k = 0; k < 4; k++) {
            uint4 v = cp[k];
            in[4 * k] = v.x;
            in[4 * k + 1] = v.y;
            in[4 * k + 2] = v.z;
            in[4 * k + 3] = v.w;
        }
        constexpr int NOUT = 2 * BITS;  // dwords for 64 codes
        uint32_t out[NOUT];
#pragma unroll
        for (int k = 0; k < NOUT; k++) out[k] = 0;
#pragma unroll
        for (int k = 0; k < 64; k++) {
            const uint32_t code = (in[k >> 2] >> (8 * (k & 3))) & 0xffu;
            const int bit = k * BITS;
            const int wd = bit >> 5, off = bit & 31;
            out[wd] |= code << off;
            if (off + BITS > 32) out[wd + 1] |= code >> (32 - off);
        }
        uint4* op = reinterpret_cast<uint4*>(rec + (int64_t)tid * NOUT * 4);
#pragma unroll
        for (int k = 0; k < NOUT / 4; k++) op[k] = make_uint4(out[4 * k], out[4 * k + 1], out[4 * k + 2], out[4 * k + 3]);
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
    __shared__ __attribute__((aligned(16))) float bvec[D];
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
        quantize_tile<D, T, KB, false>(kpool + tile_off, krec + ((int64_t)dp * H + h) * REC, smem, bvec, n_iters);
    } else if constexpr (HASV) {
        constexpr int REC = T * D * VB / 8 + 4 * T + 2 * D;
        quantize_tile<D, T, VB, true>(vpool + tile_off, vrec + ((int64_t)dp * H + h) * REC, smem, bvec, n_iters);
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
