// Instantiates the decode-attention kernels for keys without scalar codes (sign sketch only).
#include "tq_attend_kernels.h"

namespace tq {
namespace attn {

TQ_ATTN_DISPATCH(0) { return qjl ? dispatch_v<0, true>(a, vb, G, n_slices, B, s, e0, e1) : hipErrorInvalidValue; }

}  // namespace attn
}  // namespace tq
