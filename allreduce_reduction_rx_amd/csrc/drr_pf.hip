// drr_pf.hip -- instantiates the prefetching whole-tile dequantize-reduce-
// requantize kernels (k_drr_pf): codes only in the 16 x 1 layout for 1..16
// sources, and the one-source dequantization in the 4 x 4 and 8 x 2 layouts.
#include "drr.hpp"

namespace rx {

const DrrPfFns& drr_fns_pf()
{
    static const DrrPfFns t = drr_detail::make_pf_fns();
    return t;
}

}  // namespace rx
