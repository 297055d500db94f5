// attend_pad.hip -- the decode attend's partial kernels for store head_dims
// other than 64, 128 and 256 (multiples of 16, groups of 32, binary32
// scale/zero), fp16 caches: each runs on the MFMA geometry of the next of
// those three head_dims, with the channels past its own head_dim computed
// as zeros and never stored (attend_device.h, partial_body).  The bfloat16
// set is compiled in attend_pad_bf16.hip, in parallel.
#include "attend_device.h"

namespace kivi {

hipError_t launch_attend_partial_padded(const AttendArgs& a, const AttendPlan& p, float* ws_o,
                                        float* ws_ml, hipStream_t stream) {
    if (a.bf16) return launch_attend_partial_padded_bf16(a, p, ws_o, ws_ml, stream);
    return launch_partials_padded<false>(a, p, ws_o, ws_ml, stream);
}

}  // namespace kivi
