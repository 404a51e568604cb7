// GQA decode for head_dim 256 with a code width of 3, 5 or 8 (keys or values).
#include "decode_gqa_wide.hpp"

namespace kvarn {
KVARN_GQA_WIDE_D(256)
}  // namespace kvarn
