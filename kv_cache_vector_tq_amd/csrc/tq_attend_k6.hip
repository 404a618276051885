// Instantiates the decode-attention kernels for 6-bit key codes (with and without the sign sketch).
#include "tq_attend_kernels.h"

namespace tq {
namespace attn {

TQ_ATTN_DISPATCH(6) { return dispatch_width<6>(a, kcw, qjl, vb, G, n_slices, B, pre, s, e0, e1); }

}  // namespace attn
}  // namespace tq
