// GQA decode for head_dim 512 with a code width of 3, 5 or 8 (keys or values).
#include "decode_gqa_wide.hpp"

namespace kvarn {
KVARN_GQA_WIDE_D(512)
}  // namespace kvarn
