// Instantiates the quantize kernels for 1-bit key codes (with and without the sign sketch).
#include "tq_quantize_kernels.h"

namespace tq {
namespace qk {

TQ_QUANT_DISPATCH(1) { return dispatch_width<1>(q, cb, f32, g, s, e0, e1); }

}  // namespace qk
}  // namespace tq
