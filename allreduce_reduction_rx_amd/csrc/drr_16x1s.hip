// drr_16x1s.hip -- instantiates the dequantize-reduce-requantize kernels
// for the lane layout of 16 codes per chunk, 1 chunk per lane, with the FP32
// high-precision output staged through LDS (contiguous 1 KiB stores).
#include "drr.hpp"

namespace rx {

const DrrFns& drr_fns_16x1_staged()
{
    static const DrrFns t = drr_detail::make_fns<16, 1, true>();
    return t;
}

}  // namespace rx
