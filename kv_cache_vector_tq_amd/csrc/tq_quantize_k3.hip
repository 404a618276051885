// Instantiates the quantize kernels for 3-bit key codes (with and without the sign sketch).
#include "tq_quantize_kernels.h"

namespace tq {
namespace qk {

TQ_QUANT_DISPATCH(3) { return dispatch_width<3>(q, cb, f32, g, s, e0, e1); }

}  // namespace qk
}  // namespace tq
