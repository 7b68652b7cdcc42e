// attn_wide_front.hip -- the 64-rows-per-wave kernel with query half 0's first softmax parts before the first MFMA
// (PLACE_FRONT).
#include "attn_wide.h"

namespace libattn {

template hipError_t launch_attn_wide_placed<PLACE_FRONT>(const Params& p, hipStream_t stream);

}  // namespace libattn
