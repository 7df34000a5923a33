// table_f16.hip -- instantiates every kernel shape for one element
// type and one operator (gate-first), so the six combinations compile in parallel.
#include "kernels.cuh"

namespace ggrms {

const void* pick_f16(int kernel, int vb, int lanes, int vpt, int upb) {
    return pick_type<TF16, false>(kernel, vb, lanes, vpt, upb);
}

}  // namespace ggrms
