// drr_16x1s.hip -- instantiates the dequantize-reduce-requantize kernels
// for the lane layout of 16 codes per chunk, 1 chunk per lane, with the FP32
// or BF16 high-precision output staged through LDS (contiguous 1 KiB
// stores), whole tiles only (k_drr_staged).
#include "drr.hpp"

namespace rx {

const DrrFns& drr_fns_16x1_staged(int hp_bf16)
{
    static const DrrFns f32 = drr_detail::make_staged_fns<false>();
    static const DrrFns b16 = drr_detail::make_staged_fns<true>();
    return hp_bf16 ? b16 : f32;
}

}  // namespace rx
