// Launch templates of the look-ahead stack, instantiated per weight type in
// k_la_f32.hip, k_la_f16.hip and k_la_i4.hip.
#pragma once
#include "ffn_launch.hpp"
#include "pred_body.hpp"

namespace sfnn {

// Launch A of layer l: the first gup workgroups compute their runs of FFN_l's
// up (+gate) rows (input x_l = RMSNorm(r_l) built in the prologue; h to the
// workspace), the rest the next layer's predictor stage 1 on the same x_l
// (w1_t / z / r in the arguments), a few rows each.  Separate workgroups
// rather than both kinds of work in each: the up workgroups then need no
// registers for predictor rows.
template <int WT, int ACT, int NT, int NTH, int RV, int UW>
__global__ __launch_bounds__(NTH) void k_la_up_pred1(FfnArgs fa, int gup) {
  if ((int)blockIdx.x < gup) {  // workgroup-uniform
    // the FFN's workgroups, whose rows end the layer, issue their prologue
    // ahead of the stage-1 workgroups sharing their CU (with launch B's down
    // workgroups raised the same way, 1-4% faster stacks than at equal
    // priority; the bodies lower it again once their first rows are requested)
    __builtin_amdgcn_s_setprio(3);
    up_body<WT, ACT, NT, SRC_UNION, NTH, RV, true, UW>(fa, blockIdx.x, gup);
  } else {
    p1_body<WT == WT_F32 ? WT_F32 : WT_F16, NT, NTH, RV, WT == WT_I4>(fa, blockIdx.x - gup, gridDim.x - gup);
  }
}

// Predictor-stage-1 workgroups of launch A: about SFNN_LA_P1_ROWS rows of W1^T
// each with fp16 / fp32 FFN weights, SFNN_LA_P1_ROWS_I4 with INT4 ones (at rank
// 1024: 128 and 256 workgroups; 8 rows were 1-5% faster than 4 on the fp16
// stacks at batches 1-2, 4 rows 1-2% faster than 8 on OPT-175B INT4, with the
// FFN workgroups at a raised priority; 16 rows, in two passes, lose).
#ifndef SFNN_LA_P1_ROWS
#define SFNN_LA_P1_ROWS 8
#endif
#ifndef SFNN_LA_P1_ROWS_I4
#define SFNN_LA_P1_ROWS_I4 4
#endif
inline int la_p1_groups(int r, int wt) {
  const int rows = wt == WT_I4 ? SFNN_LA_P1_ROWS_I4 : SFNN_LA_P1_ROWS;
  return r / rows > 0 ? r / rows : 1;
}

// Launch B of layer l: the first tiles * rg workgroups compute the down-
// projection work items of FFN_l (one tile of one row group each; y_l and
// r_{l+1} = r_l + y_l for the tile's columns when there is one row group),
// the next gp workgroups predict one mask word each of the next layer
// (predictor stage 2).  The two kinds carry about the same bytes (a tile of
// every listed row, or 64 rows of W2^T), so the CUs take them in any order.
// (Interleaving a tile and a word in one workgroup, with the tile's loads
// issued between the word's, measured 3% slower at OPT-6.7B batch 1 and the
// same at OPT-175B.)
#ifndef SFNN_LA_B_WAVES
#define SFNN_LA_B_WAVES 2  // waves per SIMD the launch-B kernel is built for
#endif
template <int WT, int NTD, int LPR, int PWT, int NT2, int VPL>
__global__ __launch_bounds__(512, SFNN_LA_B_WAVES) void k_la_down_pred2(DownArgs da, int tiles, Pred2Args pa) {
  constexpr int RB = VPL <= 2 ? 8 : (VPL == 4 ? 4 : 2);
  __shared__ __align__(16) float red[DownRed<WT, NTD, LPR>::floats];
  const int vb = blockIdx.x;
  const int items = tiles * da.rg;
  if (vb >= items) {  // workgroup-uniform
    pred2_body<PWT, NT2, VPL, RB>(pa, vb - items);
    return;
  }
  int tile, grp;
  __builtin_amdgcn_s_setprio(3);  // the down tiles, the launch's long pole, start ahead of stage 2
  down_item(vb, tiles, 8 / LPR, tile, grp);
  down_body<WT, NTD, LPR, CO_H, true>(da, tile, grp, red);
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
  const int grid = F.groups + (next ? la_p1_groups(next->r, WT) : 0);
  if (union_words_per_lane(F.f) == 4)
    hipLaunchKernelGGL((k_la_up_pred1<WT, ACT, NT, NTH, RV, 4>), dim3(grid), dim3(NTH), sh, s, fa, F.groups);
  else
    hipLaunchKernelGGL((k_la_up_pred1<WT, ACT, NT, NTH, RV, 16>), dim3(grid), dim3(NTH), sh, s, fa, F.groups);
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

template <int WT, int NTD, int PWT, int NT2, int VPL>
static void launch_b_lpr(const DownArgs& da, const DownShape& ds, const Pred2Args& pa, int gp, hipStream_t s) {
  const dim3 grid(ds.tiles * ds.rg + gp), blk(512);
  switch (ds.lpr) {
    case 1: hipLaunchKernelGGL((k_la_down_pred2<WT, NTD, 1, PWT, NT2, VPL>), grid, blk, 0, s, da, ds.tiles, pa); break;
    case 2: hipLaunchKernelGGL((k_la_down_pred2<WT, NTD, 2, PWT, NT2, VPL>), grid, blk, 0, s, da, ds.tiles, pa); break;
    case 4: hipLaunchKernelGGL((k_la_down_pred2<WT, NTD, 4, PWT, NT2, VPL>), grid, blk, 0, s, da, ds.tiles, pa); break;
    default: hipLaunchKernelGGL((k_la_down_pred2<WT, NTD, 8, PWT, NT2, VPL>), grid, blk, 0, s, da, ds.tiles, pa); break;
  }
}

// Down work items of launch B: 0, one row group of the narrowest tiles (y and
// the residual row written directly); else whole 128-byte lines in row
// groups aiming at this many items, their partial rows added by a sum launch
// after it.
#ifndef SFNN_LA_B_ITEMS
#define SFNN_LA_B_ITEMS 0
#endif
template <int WT, int PWT, int NT2>
static void launch_b(DownArgs da, int batch, const PredLaunch& next, hipStream_t s) {
  const int gp = next.f / 64;
  const DownShape ds = down_shape(WT, da.d, batch, SFNN_LA_B_ITEMS);
  da.rg = ds.rg;
  const Pred2Args pa = pred2_args(next, 0, next.batch);
  const int vpl = pred2_vpl(PWT, next.r);
  if (ds.nt == 1) {
    if (vpl == 1) launch_b_lpr<WT, 1, PWT, NT2, 1>(da, ds, pa, gp, s);
    else if (vpl == 2) launch_b_lpr<WT, 1, PWT, NT2, 2>(da, ds, pa, gp, s);
    else launch_b_lpr<WT, 1, PWT, NT2, 4>(da, ds, pa, gp, s);
  } else {
    if (vpl == 1) launch_b_lpr<WT, 2, PWT, NT2, 1>(da, ds, pa, gp, s);
    else if (vpl == 2) launch_b_lpr<WT, 2, PWT, NT2, 2>(da, ds, pa, gp, s);
    else launch_b_lpr<WT, 2, PWT, NT2, 4>(da, ds, pa, gp, s);
  }
  if (ds.rg > 1) (void)launch_down_sum(da, s);  // errors surface through hipGetLastError
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
