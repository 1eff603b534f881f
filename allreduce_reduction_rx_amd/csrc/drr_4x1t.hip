// drr_4x1t.hip -- instantiates the decode-size dequantize-reduce-requantize
// kernels for ranges of whole tiles (k_drr_tile1), lane layout of 4 codes
// per chunk, 1 chunk per lane.
#include "drr.hpp"

namespace rx {

const DrrFns& drr_fns_4x1_tile1()
{
    static const DrrFns t = drr_detail::make_tile1_fns<4, 1>();
    return t;
}

}  // namespace rx
