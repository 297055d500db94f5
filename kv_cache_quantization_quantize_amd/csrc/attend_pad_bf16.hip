// attend_pad_bf16.hip -- the padded partial kernels of attend_pad.hip for
// bfloat16 caches, in a translation unit of their own so they compile in
// parallel with the fp16 set.
#include "attend_device.h"

namespace kivi {

hipError_t launch_attend_partial_padded_bf16(const AttendArgs& a, const AttendPlan& p, float* ws_o,
                                             float* ws_ml, hipStream_t stream) {
    return launch_partials_padded<true>(a, p, ws_o, ws_ml, stream);
}

}  // namespace kivi
