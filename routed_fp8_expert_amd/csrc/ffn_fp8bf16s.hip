// ffn_fp8bf16s.hip -- the expert kernels and launchers of ffn.hpp for one weight
// format (kFp8Bf16s), in a translation unit of their own so the formats compile in
// parallel.
#include "ffn.hpp"

namespace moe {

MOE_FFN_FORMAT_LAUNCHERS(template, kFp8Bf16s)

}  // namespace moe
