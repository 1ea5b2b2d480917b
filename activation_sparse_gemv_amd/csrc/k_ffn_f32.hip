// The gathered FFN's launches for f32 weights.
#include "ffn_launch.hpp"

namespace sfnn {

void ffn_run_f32(const FfnLaunch& p, hipStream_t s) {
  if (p.act == ACT_RELU)
    ffn_all<WT_F32, ACT_RELU>(p, s);
  else
    ffn_all<WT_F32, ACT_REGLU>(p, s);
}

}  // namespace sfnn
