// Launch templates of the one-launch gathered FFN, instantiated per weight
// type in k_ffn_f32.hip, k_ffn_f16.hip and k_ffn_i4.hip.
#pragma once
#include "ffn_body.hpp"

namespace sfnn {

template <int WT, int ACT, int NT, int SRC, int NTH, int CPT, int UW>
__global__ __launch_bounds__(NTH) void k_ffn(FfnArgs a) {
  ffn_body<WT, ACT, NT, SRC, NTH, CPT, false, false, UW>(a, blockIdx.x, gridDim.x);
}

// Union-mask words each lane holds: 4 covers d_ff <= 16384, 16 covers 65536.
inline int union_words_per_lane(int f) { return f / 64 <= 4 * kWave ? 4 : 16; }

template <int WT, int ACT, int NT, int NTH, int CPT>
static void ffn_pass(const FfnLaunch& p, int tok0, int nt, bool first, hipStream_t s) {
  using XT = typename std::conditional<WT == WT_F32, float, f16>::type;
  const FfnArgs a = ffn_args(p, tok0, nt, first);
  const size_t sh = (size_t)NT * p.d * sizeof(XT);
  const int G = p.groups;
  if (p.src == SRC_UNION) {
    if (union_words_per_lane(p.f) == 4)
      hipLaunchKernelGGL((k_ffn<WT, ACT, NT, SRC_UNION, NTH, CPT, 4>), dim3(G), dim3(NTH), sh, s, a);
    else
      hipLaunchKernelGGL((k_ffn<WT, ACT, NT, SRC_UNION, NTH, CPT, 16>), dim3(G), dim3(NTH), sh, s, a);
  } else if (p.src == SRC_IDS) {
    hipLaunchKernelGGL((k_ffn<WT, ACT, NT, SRC_IDS, NTH, CPT, 2>), dim3(G), dim3(NTH), sh, s, a);
  } else {
    hipLaunchKernelGGL((k_ffn<WT, ACT, NT, SRC_DENSE, NTH, CPT, 2>), dim3(G), dim3(NTH), sh, s, a);
  }
}

template <int WT, int ACT, int NT, int NTH>
static void ffn_pass_cpt(const FfnLaunch& p, int cpt, int tok0, int nt, bool first, hipStream_t s) {
  if (cpt == 8)
    ffn_pass<WT, ACT, NT, NTH, 8>(p, tok0, nt, first, s);
  else if (cpt == 16)
    ffn_pass<WT, ACT, (NT > 4 ? 4 : NT), NTH, 16>(p, tok0, nt, first, s);
  else
    ffn_pass<WT, ACT, (NT > 2 ? 2 : NT), NTH, 32>(p, tok0, nt, first, s);
}

template <int WT, int ACT, int NT>
static void ffn_pass_nth(const FfnLaunch& p, const FfnShape& sh, int tok0, int nt, bool first, hipStream_t s) {
  if (sh.nth == 256)
    ffn_pass<WT, ACT, NT, 256, 8>(p, tok0, nt, first, s);  // 256 threads only when d <= 2048, CPT 8
  else
    ffn_pass_cpt<WT, ACT, NT, 512>(p, sh.cpt, tok0, nt, first, s);
}

template <int WT, int ACT>
void ffn_all(const FfnLaunch& p, hipStream_t s) {
  const FfnShape sh = ffn_shape(WT, p.d, p.batch);
  for (int tok0 = 0; tok0 < p.batch; tok0 += sh.nt) {
    const int nt = (p.batch - tok0 < sh.nt) ? (p.batch - tok0) : sh.nt;
    const bool first = tok0 == 0;
    switch (sh.nt) {
      case 1: ffn_pass_nth<WT, ACT, 1>(p, sh, tok0, nt, first, s); break;
      case 2: ffn_pass_nth<WT, ACT, 2>(p, sh, tok0, nt, first, s); break;
      case 4: ffn_pass_nth<WT, ACT, 4>(p, sh, tok0, nt, first, s); break;
      default: ffn_pass_nth<WT, ACT, 8>(p, sh, tok0, nt, first, s); break;
    }
  }
  if (p.y || p.r_out) (void)launch_sum(p, s);
}

// One weight type's entry points (k_ffn_<type>.hip).
void ffn_run_f32(const FfnLaunch& p, hipStream_t s);
void ffn_run_f16(const FfnLaunch& p, hipStream_t s);
void ffn_run_i4(const FfnLaunch& p, hipStream_t s);

}  // namespace sfnn
