// drr_8x2.hip -- instantiates the dequantize-reduce-requantize kernels
// for the lane layout of 8 codes per chunk, 2 chunks per lane.
#include "drr.hpp"

namespace rx {

const DrrFns& drr_fns_8x2()
{
    static const DrrFns t = drr_detail::make_fns<8, 2>();
    return t;
}

}  // namespace rx
