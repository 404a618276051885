// Instantiates the decode-attention kernels for 1-bit key codes (with and without the sign sketch).
#include "tq_attend_kernels.h"

namespace tq {
namespace attn {

TQ_ATTN_DISPATCH(1) { return dispatch_width<1>(a, kcw, qjl, vb, G, n_slices, B, pre, s, e0, e1); }

}  // namespace attn
}  // namespace tq
