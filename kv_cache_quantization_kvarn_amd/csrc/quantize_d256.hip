// Quantize kernels for head_dim 256.
#include "quantize_impl.hpp"

namespace kvarn {
KVARN_QUANTIZE_INSTANTIATE_D(256)
}  // namespace kvarn
