// Merge of split-K decode partials, shared by the GQA and MLA decodes.
#pragma once

#include <math.h>

#include <type_traits>

#include "kvarn_device.hpp"

namespace kvarn {
namespace {

// Merge of the split partials of one (query row, head): the first nq are
// quantized-page splits with rotated-basis value sums, the rest fp16 slots
// with original-basis ones; the record part is rotated back once, the fp16
// part added, the sum normalized.  Lane l holds channels CPL l .. CPL l +
// CPL - 1 (CPL = D / 64).  The partials' maxima and weight sums meet through
// wave reductions; the value sums stream through, each split's weight read
// from the lane that owns the split (v_readlane), U of them a step (their
// loads in flight together); the inverse rotation is an
// in-register fast Walsh-Hadamard transform: in-lane stages over the low
// channel bits, then one cross-lane stage per lane bit.  With many rows each
// of a workgroup's 4 waves takes a row of its own (no LDS, no barrier); with
// few (wpr = 4) the 4 waves share one row, each taking every 4th group of
// 8 splits, and meet once in LDS before wave 0 rotates and stores.
template <int D>
__global__ void __launch_bounds__(256) split_merge_kernel(const float* __restrict__ ws, float* __restrict__ out,
                                                          int nrows, int nq, int np, int wpr) {
    constexpr int WS = D + 4;           // partial: m, l, pad, pad, value sums
    constexpr int CPL = D / 64;
    constexpr int U = CPL == 8 ? 8 : 16;  // splits per step, their loads issued together
    static_assert(CPL == 2 || CPL == 4 || CPL == 8, "head dims 128, 256, 512");
    __shared__ float red[3][2 * D + 1];  // waves 1..3 of a shared row: r, pl, Ls
    const int wave = (int)(threadIdx.x >> 6);
    const int row = wpr == 1 ? (int)blockIdx.x * 4 + wave : (int)blockIdx.x;
    const int part = wpr == 1 ? 0 : wave;   // this wave's share of the row's split groups
    if (row >= nrows) return;  // whole waves (wpr = 4: the whole workgroup)
    const int lane = threadIdx.x & 63;
    const float* base = ws + (int64_t)row * np * WS;
    // maxima and weight sums of the first 64 partials, kept for the weights
    float m0 = -INFINITY, l0 = 0.f;
    if (lane < np) {
        m0 = base[(int64_t)lane * WS];
        l0 = base[(int64_t)lane * WS + 1];
    }
    float M = m0;
    for (int s = 64 + lane; s < np; s += 64) M = fmaxf(M, base[(int64_t)s * WS]);
    M = wave_max_all(M);
    float r[CPL], pl[CPL];
#pragma unroll
    for (int c = 0; c < CPL; c++) r[c] = pl[c] = 0.f;
    float Ls = 0.f;
    if (M != -INFINITY) {  // uniform over the row; empty splits (m = -inf) weigh 0
        for (int s0 = 0; s0 < np; s0 += 64) {
            float e = 0.f;
            if (s0 + lane < np) {
                const float ms = s0 == 0 ? m0 : base[(int64_t)(s0 + lane) * WS];
                e = ms == -INFINITY ? 0.f : exp2f(ms - M);
                if (part == 0) Ls = fmaf(s0 == 0 ? l0 : base[(int64_t)(s0 + lane) * WS + 1], e, Ls);
            }
            const int n = min(64, np - s0);
            // a loop holding v_readlane is not unrolled by the compiler: U
            // splits a step by hand, slots past the end with weight 0 re-reading
            // the last split
            for (int k = U * part; k < n; k += U * wpr) {
                float v[U][CPL], er[U], ep[U];
#pragma unroll
                for (int u = 0; u < U; u++) {
                    const int kk = k + u;
                    const bool ok = kk < n;  // uniform
                    const float ek = ok ? i2f(__builtin_amdgcn_readlane(f2i(e), kk & 63)) : 0.f;
                    const bool rot = s0 + kk < nq;
                    er[u] = rot ? ek : 0.f;
                    ep[u] = rot ? 0.f : ek;
                    const float* p = base + (int64_t)(s0 + (ok ? kk : n - 1)) * WS + 4 + CPL * lane;
                    if constexpr (CPL == 2) {
                        const float2 t = *reinterpret_cast<const float2*>(p);
                        v[u][0] = t.x; v[u][1] = t.y;
                    } else {
#pragma unroll
                        for (int q = 0; q < CPL / 4; q++) {
                            const float4 t = reinterpret_cast<const float4*>(p)[q];
                            v[u][4 * q] = t.x; v[u][4 * q + 1] = t.y; v[u][4 * q + 2] = t.z; v[u][4 * q + 3] = t.w;
                        }
                    }
                }
#pragma unroll
                for (int u = 0; u < U; u++)
#pragma unroll
                    for (int c = 0; c < CPL; c++) {
                        r[c] = fmaf(er[u], v[u][c], r[c]);
                        pl[c] = fmaf(ep[u], v[u][c], pl[c]);
                    }
            }
        }
        Ls = wave_sum_all(Ls);
    }
    if (wpr > 1) {  // uniform over the workgroup
        if (wave > 0) {
#pragma unroll
            for (int c = 0; c < CPL; c++) {
                red[wave - 1][CPL * lane + c] = r[c];
                red[wave - 1][D + CPL * lane + c] = pl[c];
            }
        }
        __syncthreads();
        if (wave > 0) return;
#pragma unroll
        for (int w = 0; w < 3; w++)
#pragma unroll
            for (int c = 0; c < CPL; c++) {
                r[c] += red[w][CPL * lane + c];
                pl[c] += red[w][D + CPL * lane + c];
            }
    }
    // inverse rotation of the record part: pairs (j, j + hs) -> (a + b, a - b)
#pragma unroll
    for (int hs = 1; hs < CPL; hs <<= 1)
#pragma unroll
        for (int c = 0; c < CPL; c++)
            if (!(c & hs)) {
                const float a = r[c], b = r[c + hs];
                r[c] = a + b;
                r[c + hs] = a - b;
            }
    auto cross = [&](auto bit) {  // channel bit log2(CPL) + BIT = lane bit BIT
        constexpr int BIT = decltype(bit)::value;
        const bool hi = (lane >> BIT) & 1;
#pragma unroll
        for (int c = 0; c < CPL; c++) {
            float pv;
            if constexpr (BIT < 5) pv = xor_lane<BIT>(r[c]);
            else pv = lane_bcast32(r[c]);
            r[c] = hi ? pv - r[c] : r[c] + pv;
        }
    };
    cross(std::integral_constant<int, 0>{});
    cross(std::integral_constant<int, 1>{});
    cross(std::integral_constant<int, 2>{});
    cross(std::integral_constant<int, 3>{});
    cross(std::integral_constant<int, 4>{});
    cross(std::integral_constant<int, 5>{});
    const float rs = 1.0f / sqrtf((float)D);
    const float il = Ls > 0.f ? 1.0f / Ls : 0.f;
    float o[CPL];
#pragma unroll
    for (int c = 0; c < CPL; c++) o[c] = Ls > 0.f ? fmaf(r[c], rs, pl[c]) * il : 0.f;
    float* dst = out + (int64_t)row * D + CPL * lane;
    if constexpr (CPL == 2) {
        *reinterpret_cast<float2*>(dst) = make_float2(o[0], o[1]);
    } else {
#pragma unroll
        for (int q = 0; q < CPL / 4; q++)
            reinterpret_cast<float4*>(dst)[q] = make_float4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
    }
}

// rows (query row, head) of np partials each at `partials`, D + 4 floats a
// partial (m, l, pad, pad, value sums); the first nq hold rotated-basis sums
template <int D>
hipError_t launch_split_merge(const float* partials, float* out, int rows, int nq, int np, hipStream_t st) {
    // fewer rows than fill the chip at one wave each: four waves per row
    const int wpr = rows < 2048 ? 4 : 1;
    const int blocks = wpr == 1 ? (rows + 3) / 4 : rows;
    hipLaunchKernelGGL((split_merge_kernel<D>), dim3(blocks), dim3(256), 0, st, partials, out, rows, nq, np, wpr);
    return hipGetLastError();
}

}  // namespace
}  // namespace kvarn
