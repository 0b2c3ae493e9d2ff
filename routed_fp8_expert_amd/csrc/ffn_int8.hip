// ffn_int8.hip -- the expert kernels and launchers of ffn.hpp for one weight
// format (kInt8Row), in a translation unit of their own so the formats compile in
// parallel.
#include "ffn.hpp"

namespace moe {

MOE_FFN_FORMAT_LAUNCHERS(template, kInt8Row)

}  // namespace moe
