// table_f16_nbg.hip -- instantiates every kernel shape for one element
// type and one operator (norm-before-gate), with and without the streaming
// hint, so the six combinations compile in parallel.
#include "ggrms_kernels.hpp"

namespace ggrms {

const void* pick_f16_nbg(int kernel, int vb, int pb, int lanes, int vpt, int upb, bool nt) {
    return nt ? pick_type<TF16, true, true>(kernel, vb, pb, lanes, vpt, upb)
              : pick_type<TF16, true, false>(kernel, vb, pb, lanes, vpt, upb);
}

}  // namespace ggrms
