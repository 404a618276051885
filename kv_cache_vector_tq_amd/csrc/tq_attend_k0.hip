// Instantiates the decode-attention kernels for keys without scalar codes (sign sketch only).
#include "tq_attend_kernels.h"

namespace tq {
namespace attn {

TQ_ATTN_DISPATCH(0) { return dispatch_width<0>(a, kcw, qjl, vb, G, n_slices, B, pre, s, e0, e1); }

}  // namespace attn
}  // namespace tq
