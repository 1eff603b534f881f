// drr_4x1.hip -- instantiates the dequantize-reduce-requantize kernels
// for the lane layout of 4 codes per chunk, 1 chunk per lane.
#include "drr.hpp"

namespace rx {

const DrrFns& drr_fns_4x1()
{
    static const DrrFns t = drr_detail::make_fns<4, 1>();
    return t;
}

}  // namespace rx
