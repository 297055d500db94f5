// attend_bf16.hip -- the decode attend's partial kernels for bfloat16 caches
// (q, residual rows and the in-register reconstruction in bfloat16, MFMA on
// bfloat16 operands), in a translation unit of their own so they compile in
// parallel with the fp16 set in attend.hip.  The plan and the combine kernel
// are shared (attend.hip).
#include "attend_device.h"

namespace kivi {

hipError_t launch_attend_partial_bf16(const AttendArgs& a, const AttendPlan& p, float* ws_o,
                                      float* ws_ml, hipStream_t stream) {
    return launch_partials<4, true>(a, p, ws_o, ws_ml, stream);
}

}  // namespace kivi
