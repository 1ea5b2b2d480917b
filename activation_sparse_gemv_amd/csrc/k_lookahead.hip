// Look-ahead stack: DejaVu's asynchronous predictor, which predicts the next
// layer's sparsity one step ahead so that prediction leaves the critical path
// (53ai.com sparsity survey, DejaVu section 如何充分利用结构化稀疏进行加速).
// Layer l+1's predictor reads layer l's input x_l, so its two stages share
// launches with layer l's FFN and sum:
//   launch A(l): FFN_l's up (+gate) rows (x_l = RMSNorm(r_l) built in every
//                workgroup's prologue) + predictor stage 1 of layer l+1 on
//                the same x_l;
//   launch B(l): FFN_l's column-tiled down projection (y_l and
//                r_{l+1} = r_l + y_l, no partial rows) + predictor stage 2 of
//                layer l+1 (mask, union).
// Two launches per layer instead of four, and the predictor's weight stream
// overlaps the FFN's.  Layer 0's mask comes from its own input.
#include "la_launch.hpp"

namespace sfnn {

// The fused path handles token groups of 1 or 2 (decode batches 1 and 2);
// larger batches run the same schedule as separate launches.
static int la_group(const FfnLaunch& F, const PredLaunch& P) {
  const FfnShape sh = ffn_shape(F.wt, F.d, F.batch);
  if (F.batch > 2 || ffn_uses_mfma(F)) return 0;
  int nt = F.batch;
  if (sh.nt < nt) nt = sh.nt;
  const int pwt = F.wt == WT_F32 ? WT_F32 : WT_F16;
  if (pred2_group(pwt, P.r, F.batch) < F.batch || pred2_vpl(pwt, P.r) > 4) return 0;
  if (nt * sh.rv > kChainMaxV || F.d > 4 * sh.rv * sh.nth) return 0;  // residual rows must fit the prologue's registers
  return nt;
}

hipError_t launch_stack_lookahead(const PredLaunch* P, const FfnLaunch* F, const float* const* R, int L, float eps,
                                  float* rtmp, const char* dense, hipStream_t s) {
  auto sparse = [&](int l) { return !dense || !dense[l]; };
  hipError_t e = hipSuccess;
  if (sparse(0)) {
    // layer 0 predicts from its own input
    PredLaunch P0 = P[0];
    P0.norm.r_in = R[0];
    P0.norm.x_out = const_cast<void*>(F[0].x);
    P0.norm.eps = eps;
    e = launch_predict(P0, s);
    if (e != hipSuccess) return e;
  }
  // the fused launches pair every layer with the next one's predictor, so a
  // stack with dense layers takes the per-stage schedule below
  const int NT = dense ? 0 : la_group(F[0], P[0]);
  if (NT > 0) {
    if (F[0].wt == WT_F32)
      stack_fused_f32(P, F, R, L, eps, NT, s);
    else if (F[0].wt == WT_F16)
      stack_fused_f16(P, F, R, L, eps, NT, s);
    else
      stack_fused_i4(P, F, R, L, eps, NT, s);
    return hipGetLastError();
  }
  // larger batches: the same schedule, one launch per stage; a dense layer
  // has no predictor stages, and the layer before it builds x_l on its own
  for (int l = 0; l < L; ++l) {
    const bool next_predicts = l + 1 < L && sparse(l + 1);
    if (next_predicts) {
      PredLaunch Pn = P[l + 1];  // stage 1 of the next layer also writes x_l for this layer's FFN
      Pn.norm.r_in = R[l];
      Pn.norm.x_out = const_cast<void*>(F[l].x);
      Pn.norm.eps = eps;
      e = launch_predict_stage1(Pn, s);
    } else {
      // RMSNorm of the residual row alone (the row copy goes to rtmp)
      e = launch_residual_rmsnorm(R[l], nullptr, rtmp, F[l].batch, F[l].d, eps, const_cast<void*>(F[l].x),
                              F[l].wt == WT_F32 ? WT_F32 : WT_F16, s);
    }
    FfnLaunch Fs = F[l];  // y_l, and r_{l+1} = r_l + y_l
    Fs.r_in = R[l];
    Fs.r_out = const_cast<float*>(R[l + 1]);
    if (e == hipSuccess) e = launch_ffn(Fs, s);
    if (e == hipSuccess && next_predicts) e = launch_predict_stage2(P[l + 1], s);
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

}  // namespace sfnn
