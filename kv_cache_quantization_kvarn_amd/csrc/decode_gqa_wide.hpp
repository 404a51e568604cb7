// GQA decode for code widths 3, 5 and 8: the launcher, included only by the
// per-head-dim sources decode_gqa_w<D>.hip that instantiate it.
#pragma once

#include "decode_gqa_impl.hpp"

namespace kvarn {

// Code widths 3, 5 and 8 at any head dim (and every pair at head_dim 256 and
// 512): the queries rotated once by qrot_kernel, the fp16-MFMA split kernel,
// the combine.  Explicitly instantiated per head dim in decode_gqa_w<D>.hip.
template <int D, int T, int KB, int VB>
hipError_t launch_gqa_wide(const DecodeArgs& a, hipStream_t st) {
    hipLaunchKernelGGL((qrot_kernel<D>), dim3(a.B * a.Hq), dim3(D / 2), 0, st, a.q, a.q_dtype, a.ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    constexpr int NWV = split_waves<D>();
    const int nfx = (a.nfsplit + NWV - 1) / NWV;  // fp16 slots: one per wave
    const int gy = a.H * a.GS;
    const dim3 grid(split_grid_x(a.nsplit > nfx ? a.nsplit : nfx, gy, a.M, a.GS), gy, a.nfsplit > 0 ? 2 * a.B : a.B);
    hipLaunchKernelGGL((decode_split_kernel<D, T, KB, VB>), grid, dim3(64 * NWV), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_combine<D>(a, st);
}

// every (K, V) width pair with a width of 3, 5 or 8, for tiles of T tokens
#define KVARN_GQA_WIDE_K(D, T, KB)                                                                           \
    template hipError_t launch_gqa_wide<D, T, KB, 2>(const DecodeArgs&, hipStream_t);                        \
    template hipError_t launch_gqa_wide<D, T, KB, 3>(const DecodeArgs&, hipStream_t);                        \
    template hipError_t launch_gqa_wide<D, T, KB, 4>(const DecodeArgs&, hipStream_t);                        \
    template hipError_t launch_gqa_wide<D, T, KB, 5>(const DecodeArgs&, hipStream_t);                        \
    template hipError_t launch_gqa_wide<D, T, KB, 6>(const DecodeArgs&, hipStream_t);                        \
    template hipError_t launch_gqa_wide<D, T, KB, 8>(const DecodeArgs&, hipStream_t);
#define KVARN_GQA_WIDE_ODDV(D, T, KB)                                                                        \
    template hipError_t launch_gqa_wide<D, T, KB, 3>(const DecodeArgs&, hipStream_t);                        \
    template hipError_t launch_gqa_wide<D, T, KB, 5>(const DecodeArgs&, hipStream_t);                        \
    template hipError_t launch_gqa_wide<D, T, KB, 8>(const DecodeArgs&, hipStream_t);
#define KVARN_GQA_WIDE_T(D, T)                                                                               \
    KVARN_GQA_WIDE_K(D, T, 3) KVARN_GQA_WIDE_K(D, T, 5) KVARN_GQA_WIDE_K(D, T, 8)                            \
    KVARN_GQA_WIDE_ODDV(D, T, 2) KVARN_GQA_WIDE_ODDV(D, T, 4) KVARN_GQA_WIDE_ODDV(D, T, 6)
#define KVARN_GQA_WIDE_D(D) KVARN_GQA_WIDE_T(D, 128) KVARN_GQA_WIDE_T(D, 64)

}  // namespace kvarn
