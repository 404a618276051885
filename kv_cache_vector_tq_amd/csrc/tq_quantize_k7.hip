// Instantiates the quantize kernels for 7-bit key codes (with and without the sign sketch).
#include "tq_quantize_kernels.h"

namespace tq {
namespace qk {

TQ_QUANT_DISPATCH(7) { return dispatch_width<7>(q, cb, f32, g, s, e0, e1); }

}  // namespace qk
}  // namespace tq
