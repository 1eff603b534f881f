// drr_16x1.hip -- instantiates the dequantize-reduce-requantize kernels
// for the lane layout of 16 codes per chunk, 1 chunk per lane.
#include "drr.hpp"

namespace rx {

const DrrFns& drr_fns_16x1()
{
    static const DrrFns t = drr_detail::make_fns<16, 1>();
    return t;
}

}  // namespace rx
