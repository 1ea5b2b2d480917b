// Launch templates of the look-ahead stack, instantiated per weight type in
// k_la_f32.hip, k_la_f16.hip and k_la_i4.hip.
#pragma once
#include "ffn_launch.hpp"
#include "pred_body.hpp"

namespace sfnn {

// Launch A of layer l: every workgroup does its share of FFN_l (input
// x_l = RMSNorm(r_l) built in its prologue) and its share of the next layer's
// predictor stage 1 on the same x_l (w1_t / z / r in the arguments; r = 0 on
// the last layer).
template <int WT, int ACT, int NT, int NTH, int CPT, int UW>
__global__ __launch_bounds__(NTH) void k_la_ffn_pred1(FfnArgs fa) {
  ffn_body<WT, ACT, NT, SRC_UNION, NTH, CPT, true, true, UW>(fa, blockIdx.x, gridDim.x);
}

// Launch B of layer l: workgroup vb sums its slice of FFN_l's partials
// (y_l, r_{l+1}) if vb < gs, and predicts mask word vb of the next layer if
// vb < gp.  The sum's loads go out first and finish after the predictor's.
template <int PWT, int NT2, int VPL>
__global__ __launch_bounds__(512) void k_la_sum_pred2(SumArgs sa, int gs, Pred2Args pa, int gp) {
  constexpr int RB = VPL <= 2 ? 8 : (VPL == 4 ? 4 : 2);
  const int vb = blockIdx.x;
  SumLoads L;
  if (vb < gs) sum_issue(sa, vb, gs, L);
  if (vb < gp) pred2_body<PWT, NT2, VPL, RB>(pa, vb);
  if (vb < gs) sum_finish(sa, vb, gs, L);
}

// Launch A for one token group.  next == null: the last layer (FFN only).
template <int WT, int ACT, int NT, int NTH, int CPT>
static void launch_a(const FfnLaunch& F, const float* r_l, float eps, const PredLaunch* next, int tok0, int nt,
                     bool first, hipStream_t s) {
  using XT = typename std::conditional<WT == WT_F32, float, f16>::type;
  FfnArgs fa = ffn_args(F, tok0, nt, first);
  fa.r_in = r_l;
  fa.x_out = const_cast<void*>(F.x);
  fa.eps = eps;
  if (next) {
    fa.w1_t = (const uint8_t*)next->w1_t;
    fa.z = next->z;
    fa.r = next->r;
  }
  const size_t sh = (size_t)NT * F.d * sizeof(XT);
  if (union_words_per_lane(F.f) == 4)
    hipLaunchKernelGGL((k_la_ffn_pred1<WT, ACT, NT, NTH, CPT, 4>), dim3(F.groups), dim3(NTH), sh, s, fa);
  else
    hipLaunchKernelGGL((k_la_ffn_pred1<WT, ACT, NT, NTH, CPT, 16>), dim3(F.groups), dim3(NTH), sh, s, fa);
}

template <int WT, int ACT, int NT>
static void launch_a_shape(const FfnLaunch& F, const FfnShape& sh, const float* r_l, float eps,
                           const PredLaunch* next, int tok0, int nt, bool first, hipStream_t s) {
  if (sh.nth == 256)
    launch_a<WT, ACT, NT, 256, 8>(F, r_l, eps, next, tok0, nt, first, s);
  else if (sh.cpt == 8)
    launch_a<WT, ACT, NT, 512, 8>(F, r_l, eps, next, tok0, nt, first, s);
  else if (sh.cpt == 16)
    launch_a<WT, ACT, NT, 512, 16>(F, r_l, eps, next, tok0, nt, first, s);
  else
    launch_a<WT, ACT, NT, 512, 32>(F, r_l, eps, next, tok0, nt, first, s);
}

template <int WT, int ACT>
static void launch_a_all(const FfnLaunch& F, int NT, const FfnShape& sh, const float* r_l, float eps,
                         const PredLaunch* next, hipStream_t s) {
  for (int tok0 = 0; tok0 < F.batch; tok0 += NT) {
    const int nt = (F.batch - tok0 < NT) ? (F.batch - tok0) : NT;
    if (NT == 1)
      launch_a_shape<WT, ACT, 1>(F, sh, r_l, eps, next, tok0, nt, tok0 == 0, s);
    else
      launch_a_shape<WT, ACT, 2>(F, sh, r_l, eps, next, tok0, nt, tok0 == 0, s);
  }
}

template <int PWT, int NT2>
static void launch_b_vpl(const SumArgs& sa, const PredLaunch& next, hipStream_t s) {
  const int gs = sum_groups(sa.B, sa.d);
  const int gp = next.f / 64;
  const Pred2Args pa = pred2_args(next, 0, next.batch);
  const dim3 grid(gs > gp ? gs : gp);
  switch (pred2_vpl(PWT, next.r)) {
    case 1: hipLaunchKernelGGL((k_la_sum_pred2<PWT, NT2, 1>), grid, dim3(512), 0, s, sa, gs, pa, gp); break;
    case 2: hipLaunchKernelGGL((k_la_sum_pred2<PWT, NT2, 2>), grid, dim3(512), 0, s, sa, gs, pa, gp); break;
    default: hipLaunchKernelGGL((k_la_sum_pred2<PWT, NT2, 4>), grid, dim3(512), 0, s, sa, gs, pa, gp); break;
  }
}

template <int WT, int ACT>
void stack_fused(const PredLaunch* P, const FfnLaunch* F, const float* const* R, int L, float eps, int NT,
                 hipStream_t s) {
  constexpr int PWT = WT == WT_F32 ? WT_F32 : WT_F16;
  const FfnShape sh = ffn_shape(WT, F[0].d, F[0].batch);
  for (int l = 0; l < L; ++l) {
    const PredLaunch* next = (l + 1 < L) ? &P[l + 1] : nullptr;
    launch_a_all<WT, ACT>(F[l], NT, sh, R[l], eps, next, s);
    FfnLaunch Fs = F[l];
    Fs.r_in = R[l];
    Fs.r_out = const_cast<float*>(R[l + 1]);
    const SumArgs sa = sum_args(Fs);
    if (next) {
      if (next->batch == 1)
        launch_b_vpl<PWT, 1>(sa, *next, s);
      else
        launch_b_vpl<PWT, 2>(sa, *next, s);
    } else {
      (void)launch_sum(Fs, s);
    }
  }
}

// One weight type's fused schedule (k_la_<type>.hip).
void stack_fused_f32(const PredLaunch* P, const FfnLaunch* F, const float* const* R, int L, float eps, int NT,
                     hipStream_t s);
void stack_fused_f16(const PredLaunch* P, const FfnLaunch* F, const float* const* R, int L, float eps, int NT,
                     hipStream_t s);
void stack_fused_i4(const PredLaunch* P, const FfnLaunch* F, const float* const* R, int L, float eps, int NT,
                    hipStream_t s);

}  // namespace sfnn
