// Instantiates the quantize kernels for keys without scalar codes (sign sketch only).
#include "tq_quantize_kernels.h"

namespace tq {
namespace qk {

TQ_QUANT_DISPATCH(0) { return dispatch_width<0>(q, cb, f32, g, s, e0, e1); }

}  // namespace qk
}  // namespace tq
