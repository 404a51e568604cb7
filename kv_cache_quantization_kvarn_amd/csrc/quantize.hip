// Dispatch of kvarn_quantize to the kernel instantiated for the layout.
#include "kvarn_internal.hpp"

namespace kvarn {
namespace {

template <int D, int T, int KB>
hipError_t by_vbits(int vb, const QuantizeArgs& a, hipStream_t st) {
    switch (vb) {
        case 2: return launch_quantize_shape<D, T, KB, 2, true>(a, st);
        case 4: return launch_quantize_shape<D, T, KB, 4, true>(a, st);
        case 6: return launch_quantize_shape<D, T, KB, 6, true>(a, st);
        default: return hipErrorInvalidValue;
    }
}

template <int D, int T, bool CHMAJOR>
hipError_t one_kind(int bits, const QuantizeArgs& a, hipStream_t st) {
    switch (bits) {
        case 2: return launch_quantize_one<D, T, 2, CHMAJOR>(a, st);
        case 3: return launch_quantize_one<D, T, 3, CHMAJOR>(a, st);
        case 4: return launch_quantize_one<D, T, 4, CHMAJOR>(a, st);
        case 5: return launch_quantize_one<D, T, 5, CHMAJOR>(a, st);
        case 6: return launch_quantize_one<D, T, 6, CHMAJOR>(a, st);
        case 8: return launch_quantize_one<D, T, 8, CHMAJOR>(a, st);
        default: return hipErrorInvalidValue;
    }
}

bool even_width(int b) { return b == 2 || b == 4 || b == 6; }

// Rope sidecar: page i's T x R fp16 rope keys, fp16 page src[i] -> record
// page dst[i], 16 bytes a thread; a pair with an id outside its pool is
// skipped (as the quantize kernel skips it).
__global__ void __launch_bounds__(256) rope_copy_kernel(const uint4* __restrict__ from, uint4* __restrict__ to,
                                                        const int32_t* __restrict__ src,
                                                        const int32_t* __restrict__ dst, int n, int units,
                                                        int64_t n_fpages, int64_t n_qpages) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)n * units) return;
    const int i = (int)(idx / units), u = (int)(idx % units);
    const int s = src[i], d = dst[i];
    if (s < 0 || (int64_t)s >= n_fpages || d < 0 || (int64_t)d >= n_qpages) return;
    to[(int64_t)d * units + u] = from[(int64_t)s * units + u];
}

hipError_t launch_rope_copy(const QuantizeArgs& a, hipStream_t st) {
    const int units = a.T * a.R * 2 / 16;  // 16-byte units of a page's rope keys
    const int64_t total = (int64_t)a.n * units;
    const int64_t blocks = (total + 255) / 256;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(rope_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                       static_cast<const uint4*>(a.rope_fp16), static_cast<uint4*>(a.rope_records), a.src, a.dst,
                       a.n, units, a.n_fpages, a.n_qpages);
    return hipGetLastError();
}

template <int D, int T>
hipError_t by_bits(const QuantizeArgs& a, hipStream_t st) {
    if (!a.mla && !(even_width(a.k_bits) && even_width(a.v_bits))) {
        // a width of 3, 5 or 8: keys and values in two launches
        const hipError_t e = one_kind<D, T, false>(a.k_bits, a, st);
        return e != hipSuccess ? e : one_kind<D, T, true>(a.v_bits, a, st);
    }
    if (a.mla) {
        if constexpr (D == 512) {
            if (a.k_bits == 4) return launch_quantize_shape<512, T, 4, 4, false>(a, st);
        }
        return hipErrorInvalidValue;
    }
    switch (a.k_bits) {
        case 2: return by_vbits<D, T, 2>(a.v_bits, a, st);
        case 4: return by_vbits<D, T, 4>(a.v_bits, a, st);
        case 6: return by_vbits<D, T, 6>(a.v_bits, a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_quantize(const QuantizeArgs& a, hipStream_t st) {
    if (a.n == 0) return hipSuccess;
    hipError_t e = hipErrorInvalidValue;
    if (a.D == 128 && a.T == 128) e = by_bits<128, 128>(a, st);
    else if (a.D == 128 && a.T == 64) e = by_bits<128, 64>(a, st);
    else if (a.D == 256 && a.T == 128) e = by_bits<256, 128>(a, st);
    else if (a.D == 256 && a.T == 64) e = by_bits<256, 64>(a, st);
    else if (a.D == 512 && a.T == 128) e = by_bits<512, 128>(a, st);
    else if (a.D == 512 && a.T == 64) e = by_bits<512, 64>(a, st);
    if (e != hipSuccess || a.R == 0) return e;
    return launch_rope_copy(a, st);
}

}  // namespace kvarn
