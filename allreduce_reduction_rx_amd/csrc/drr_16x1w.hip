// drr_16x1w.hip -- instantiates the whole-tile dequantize-reduce-requantize
// kernels (k_drr_whole) for the lane layout of 16 codes per chunk, 1 chunk
// per lane, 1..16 sources.
#include "drr.hpp"

namespace rx {

const DrrFns& drr_fns_16x1_whole()
{
    static const DrrFns t = drr_detail::make_whole_fns<16, 1>();
    return t;
}

}  // namespace rx
