// Quantize kernels for head_dim 512 and the 512-wide MLA latent (int4, keys only).
#include "quantize_impl.hpp"

namespace kvarn {
KVARN_QUANTIZE_INSTANTIATE_D(512)
template hipError_t launch_quantize_shape<512, 128, 4, 4, false>(const QuantizeArgs&, hipStream_t);
template hipError_t launch_quantize_shape<512, 64, 4, 4, false>(const QuantizeArgs&, hipStream_t);
}  // namespace kvarn
