// attn_wide_even.hip -- the 64-rows-per-wave kernel with the softmax parts
// spread evenly (PLACE_EVEN), its grid size, and the launch by placement.
#include "attn_wide.h"

namespace libattn {

template hipError_t launch_attn_wide_placed<PLACE_EVEN>(const Params& p, hipStream_t stream);
extern template hipError_t launch_attn_wide_placed<PLACE_FRONT>(const Params& p, hipStream_t stream);
extern template hipError_t launch_attn_wide_placed<PLACE_EARLY>(const Params& p, hipStream_t stream);

int64_t grid_blocks_wide(const Params& p) {
  const int64_t nb = (int64_t)p.B * p.Hkv * p.pairs * p.n_qt;
  return nb > 0x7fffffff ? -1 : nb;
}

hipError_t launch_attn_wide(const Params& p, hipStream_t stream) {
  switch (p.place) {
    case PLACE_EVEN: return launch_attn_wide_placed<PLACE_EVEN>(p, stream);
    case PLACE_FRONT: return launch_attn_wide_placed<PLACE_FRONT>(p, stream);
    case PLACE_EARLY: return launch_attn_wide_placed<PLACE_EARLY>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace libattn
