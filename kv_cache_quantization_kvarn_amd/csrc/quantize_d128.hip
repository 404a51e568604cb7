// Quantize kernels for head_dim 128.
#include "quantize_impl.hpp"

namespace kvarn {
KVARN_QUANTIZE_INSTANTIATE_D(128)
}  // namespace kvarn
