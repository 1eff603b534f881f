// drr_4x4.hip -- instantiates the dequantize-reduce-requantize kernels
// for the lane layout of 4 codes per chunk, 4 chunks per lane.
#include "drr.hpp"

namespace rx {

const DrrFns& drr_fns_4x4()
{
    static const DrrFns t = drr_detail::make_fns<4, 4>();
    return t;
}

}  // namespace rx
