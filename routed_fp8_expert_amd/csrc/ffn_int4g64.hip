// ffn_int4g64.hip -- the expert kernels and launchers of ffn.hpp for one weight
// format (kInt4G64), in a translation unit of their own so the formats compile in
// parallel.
#include "ffn.hpp"

namespace moe {

MOE_FFN_FORMAT_LAUNCHERS(template, kInt4G64)

}  // namespace moe
