// table_f16.hip -- instantiates every kernel shape for one element
// type and one operator (gate-first), with and without the streaming hint,
// so the six combinations compile in parallel.
#include "ggrms_kernels.hpp"

namespace ggrms {

const void* pick_f16(int kernel, int vb, int pb, int lanes, int vpt, int upb, bool nt) {
    return nt ? pick_type<TF16, false, true>(kernel, vb, pb, lanes, vpt, upb)
              : pick_type<TF16, false, false>(kernel, vb, pb, lanes, vpt, upb);
}

}  // namespace ggrms
