// Instantiates the decode-attention kernels for 1-bit key codes (with and without the sign sketch).
#include "tq_attend_kernels.h"

namespace tq {
namespace attn {

TQ_ATTN_DISPATCH(1) { return qjl ? dispatch_v<1, true>(a, vb, G, n_slices, B, pre, s, e0, e1) : dispatch_v<1, false>(a, vb, G, n_slices, B, pre, s, e0, e1); }

}  // namespace attn
}  // namespace tq
