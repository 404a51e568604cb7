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
    if (a.D == 128 && a.T == 128) return by_bits<128, 128>(a, st);
    if (a.D == 128 && a.T == 64) return by_bits<128, 64>(a, st);
    if (a.D == 256 && a.T == 128) return by_bits<256, 128>(a, st);
    if (a.D == 256 && a.T == 64) return by_bits<256, 64>(a, st);
    if (a.D == 512 && a.T == 128) return by_bits<512, 128>(a, st);
    if (a.D == 512 && a.T == 64) return by_bits<512, 64>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace kvarn
