// attn_wide_early.hip -- the 64-rows-per-wave kernel with query half 1's softmax parts ending four steps early
// (PLACE_EARLY).
#include "attn_wide.h"

namespace libattn {

template hipError_t launch_attn_wide_placed<PLACE_EARLY>(const Params& p, hipStream_t stream);

}  // namespace libattn
