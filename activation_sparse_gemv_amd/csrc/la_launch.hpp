// Launch templates of the look-ahead stack, instantiated per weight type in
// k_la_f32.hip, k_la_f16.hip and k_la_i4.hip.
#pragma once
#include "ffn_launch.hpp"
#include "pred_body.hpp"

namespace sfnn {

// Launch A of layer l: every workgroup computes its run of FFN_l's up (+gate)
// rows (input x_l = RMSNorm(r_l) built in its prologue; h to the workspace)
// and its share of the next layer's predictor stage 1 on the same x_l
// (w1_t / z / r in the arguments; r = 0 on the last layer).
template <int WT, int ACT, int NT, int NTH, int RV, int UW>
__global__ __launch_bounds__(NTH) void k_la_up_pred1(FfnArgs fa) {
  up_body<WT, ACT, NT, SRC_UNION, NTH, RV, true, true, UW>(fa, blockIdx.x, gridDim.x);
}

// Launch B of layer l: workgroup vb predicts mask word vb of the next layer
// if vb < gp, and computes down-projection work item vb of FFN_l (one tile of
// one row group; y_l and r_{l+1} = r_l + y_l for the tile's columns once its
// row groups are in) if vb < tiles * row groups.  A workgroup with an item
// interleaves the two streams: the item's row ids, then the predictor's z and
// W2^T rows, then the item's first weights, then the predictor's math (whose
// waits stop short of those weights), then the rest of the item; its loads
// sit in no branch (with no word of its own it reads the last word's rows and
// writes nothing).  A workgroup without an item only predicts (an early exit,
// so the item path stays branch-free).  With a dense hot prefix (HOT) a word
// may need no loads at all, and the two parts run one after the other.
template <int WT, int NTD, int LPR, int PWT, int NT2, int VPL, bool HOT>
#ifndef SFNN_LA_B_WAVES
#define SFNN_LA_B_WAVES 2  // waves per SIMD the launch-B kernel is built for (4 would force two workgroups per CU: spills)
#endif
__global__ __launch_bounds__(512, SFNN_LA_B_WAVES) void k_la_down_pred2(DownArgs da, int tiles, Pred2Args pa,
                                                                         int gp) {
  constexpr int RB = VPL <= 2 ? 8 : (VPL == 4 ? 4 : 2);
  __shared__ __align__(16) float red[DownRed<WT, NTD, LPR>::floats];
  const int vb = blockIdx.x;
  if (vb >= tiles * da.rg) {  // workgroup-uniform
    pred2_body<PWT, NT2, VPL, RB>(pa, vb);  // vb < gp: the grid is max(items, gp)
    return;
  }
  const bool hasp = vb < gp;
  DownTile<WT, NTD, LPR, CO_H, true> D;
  int tile, grp;
  down_item(vb, tiles, 8 / LPR, tile, grp);
  D.count(da, tile, grp, true);
  if constexpr (HOT) {
    if (hasp) pred2_body<PWT, NT2, VPL, RB>(pa, vb);
    D.ids01(da);
    D.first(da);
    D.loop(da);
  } else {
    D.ids01(da);
    Pred2Tile<PWT, NT2, VPL, RB> P;
    const int vp = hasp ? vb : gp - 1;
    P.issue(pa, vp);
    D.first(da);
    P.finish(pa, vp, hasp);
    D.loop(da);
  }
  D.finish(da, red, true);
}

// Launch A for one token group.  next == null: the last layer (FFN only).
template <int WT, int ACT, int NT, int RV>
static void launch_a(const FfnLaunch& F, const float* r_l, float eps, const PredLaunch* next, int tok0, int nt,
                     bool first, hipStream_t s) {
  using XT = typename std::conditional<WT == WT_F32, float, f16>::type;
  constexpr int NTH = 512;
  FfnArgs fa = ffn_args(F, tok0, nt, first);
  fa.r_in = r_l;
  fa.x_out = const_cast<void*>(F.x);
  fa.eps = eps;
  if (next) {
    fa.w1_t = (const uint8_t*)next->w1_t;
    fa.z = next->z;
    fa.r = next->r;
  }
  const size_t sh = (size_t)NT * F.d * sizeof(XT) + (WT == WT_I4 ? (size_t)NT * (F.d / 32) * 4 : 0);  // + vec_i4's m8
  if (union_words_per_lane(F.f) == 4)
    hipLaunchKernelGGL((k_la_up_pred1<WT, ACT, NT, NTH, RV, 4>), dim3(F.groups), dim3(NTH), sh, s, fa);
  else
    hipLaunchKernelGGL((k_la_up_pred1<WT, ACT, NT, NTH, RV, 16>), dim3(F.groups), dim3(NTH), sh, s, fa);
}

template <int WT, int ACT, int NT>
static void launch_a_shape(const FfnLaunch& F, const FfnShape& sh, const float* r_l, float eps,
                           const PredLaunch* next, int tok0, int nt, bool first, hipStream_t s) {
  if (sh.rv == 2)
    launch_a<WT, ACT, NT, 2>(F, r_l, eps, next, tok0, nt, first, s);
  else if (sh.rv == 4)
    launch_a<WT, ACT, NT, 4>(F, r_l, eps, next, tok0, nt, first, s);
  else
    launch_a<WT, ACT, NT, 8>(F, r_l, eps, next, tok0, nt, first, s);
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

template <int WT, int NTD, int PWT, int NT2, int VPL, bool HOT>
static void launch_b_lpr(const DownArgs& da, const DownShape& ds, const Pred2Args& pa, int gp, hipStream_t s) {
  const int items = ds.tiles * ds.rg;
  const dim3 grid(items > gp ? items : gp), blk(512);
  switch (ds.lpr) {
    case 1: hipLaunchKernelGGL((k_la_down_pred2<WT, NTD, 1, PWT, NT2, VPL, HOT>), grid, blk, 0, s, da, ds.tiles, pa, gp); break;
    case 2: hipLaunchKernelGGL((k_la_down_pred2<WT, NTD, 2, PWT, NT2, VPL, HOT>), grid, blk, 0, s, da, ds.tiles, pa, gp); break;
    case 4: hipLaunchKernelGGL((k_la_down_pred2<WT, NTD, 4, PWT, NT2, VPL, HOT>), grid, blk, 0, s, da, ds.tiles, pa, gp); break;
    default: hipLaunchKernelGGL((k_la_down_pred2<WT, NTD, 8, PWT, NT2, VPL, HOT>), grid, blk, 0, s, da, ds.tiles, pa, gp); break;
  }
}

template <int WT, int NTD, int PWT, int NT2, int VPL>
static void launch_b_hot(const DownArgs& da, const DownShape& ds, const Pred2Args& pa, int gp, hipStream_t s) {
  if (pa.hot > 0)
    launch_b_lpr<WT, NTD, PWT, NT2, VPL, true>(da, ds, pa, gp, s);
  else
    launch_b_lpr<WT, NTD, PWT, NT2, VPL, false>(da, ds, pa, gp, s);
}

// Launch B: the down projection of this layer (every token, batch <= 2) and
// the next layer's predictor stage 2.
// Down work items launch B aims at (0: one row group of narrow tiles, the
// tiles' workgroups each also predicting a word).
#ifndef SFNN_LA_B_ITEMS
#define SFNN_LA_B_ITEMS 0
#endif
constexpr int kLaBItems = SFNN_LA_B_ITEMS;

template <int WT, int PWT, int NT2>
static void launch_b(DownArgs da, int batch, const PredLaunch& next, hipStream_t s) {
  const int gp = next.f / 64;
  const DownShape ds = down_shape(WT, da.d, batch, kLaBItems);
  da.rg = ds.rg;
  const Pred2Args pa = pred2_args(next, 0, next.batch);
  const int vpl = pred2_vpl(PWT, next.r);
  if (ds.nt == 1) {
    if (vpl == 1) launch_b_hot<WT, 1, PWT, NT2, 1>(da, ds, pa, gp, s);
    else if (vpl == 2) launch_b_hot<WT, 1, PWT, NT2, 2>(da, ds, pa, gp, s);
    else launch_b_hot<WT, 1, PWT, NT2, 4>(da, ds, pa, gp, s);
  } else {
    if (vpl == 1) launch_b_hot<WT, 2, PWT, NT2, 1>(da, ds, pa, gp, s);
    else if (vpl == 2) launch_b_hot<WT, 2, PWT, NT2, 2>(da, ds, pa, gp, s);
    else launch_b_hot<WT, 2, PWT, NT2, 4>(da, ds, pa, gp, s);
  }
  if (ds.rg > 1) launch_down_sum(da, s);
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
    const DownArgs da = ffn_down_args(Fs);
    if (next) {
      if (next->batch == 1)
        launch_b<WT, PWT, 1>(da, F[l].batch, *next, s);
      else
        launch_b<WT, PWT, 2>(da, F[l].batch, *next, s);
    } else {
      down_all<WT, CO_H>(da, F[l].batch, s);
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
