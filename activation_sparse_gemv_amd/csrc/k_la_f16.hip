// The look-ahead stack's fused launches for f16 FFN weights.
#include "la_launch.hpp"

namespace sfnn {

void stack_fused_f16(const PredLaunch* P, const FfnLaunch* F, const float* const* R, int L, float eps, int NT,
                        hipStream_t s) {
  if (F[0].act == ACT_RELU)
    stack_fused<WT_F16, ACT_RELU>(P, F, R, L, eps, NT, s);
  else
    stack_fused<WT_F16, ACT_REGLU>(P, F, R, L, eps, NT, s);
}

}  // namespace sfnn
