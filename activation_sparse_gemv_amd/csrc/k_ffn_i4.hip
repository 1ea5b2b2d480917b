// The gathered FFN's launches for i4 weights.
#include "ffn_launch.hpp"

namespace sfnn {

void ffn_run_i4(const FfnLaunch& p, hipStream_t s) {
  if (p.act == ACT_RELU)
    ffn_all<WT_I4, ACT_RELU>(p, s);
  else
    ffn_all<WT_I4, ACT_REGLU>(p, s);
}

}  // namespace sfnn
