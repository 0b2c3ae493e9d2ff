// ffn_nvfp4.hip -- the expert kernels and launchers of ffn.hpp for one weight
// format (kNvfp4), in a translation unit of their own so the formats compile in
// parallel.
#include "ffn.hpp"

namespace moe {

MOE_FFN_FORMAT_LAUNCHERS(template, kNvfp4)

}  // namespace moe
