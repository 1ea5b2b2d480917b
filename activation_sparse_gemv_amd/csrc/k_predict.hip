// Predictor launches: k_pred1 (z = W1^T x, optionally from the residual row)
// and k_pred2 (logits, threshold, packed masks, union).  The workgroup bodies
// live in pred_body.hpp.
#include "pred_body.hpp"

namespace sfnn {

template <int WT, int LPR, int NT, bool CHAIN>
__global__ __launch_bounds__(256) void k_pred1(Pred1Args a) {
  pred1_body<WT, LPR, NT, CHAIN>(a, blockIdx.x, gridDim.x);
}

template <int WT, int NT, int VPL, int RB>
__global__ __launch_bounds__(512) void k_pred2(Pred2Args a) {
  pred2_body<WT, NT, VPL, RB>(a, blockIdx.x);
}

static int pow2_floor(int v) {
  int p = 1;
  while (p * 2 <= v) p *= 2;
  return p;
}

static int group_for(int batch, int cap) {
  if (cap < 1) cap = 1;
  if (cap > kMaxNT) cap = kMaxNT;
  cap = pow2_floor(cap);
  int nt = 1;
  while (nt < batch && nt < cap) nt *= 2;
  return nt;
}

// Token group of stage 1: staged x in LDS, and in a residual stack the
// residual rows held in registers (256 threads).
int pred_group(int wt, int d, int r, int batch, bool chain) {
  (void)r;
  const int xb = (wt == WT_F32) ? 4 : 2;
  int cap = kStageBytes / (d * xb);
  if (chain) {
    const int cap2 = kChainMaxV * 256 * 4 / d;
    if (cap2 < cap) cap = cap2;
  }
  return group_for(batch, cap);
}

// Vectors per lane per W2^T row in stage 2.
int pred2_vpl(int wt, int r) {
  const int nvec = r * (wt == WT_F32 ? 4 : 2) / 16;
  int vpl = 1;
  while (vpl * kWave < nvec) vpl *= 2;
  return vpl;
}

// Token group of stage 2: z in registers, NT * VPL * E <= 64 floats.
int pred2_group(int wt, int r, int batch) {
  const int E = (wt == WT_F32) ? 4 : 8;
  const int vpl = pred2_vpl(wt, r);
  int g = group_for(batch, 64 / (vpl * E));
  if (vpl == 4 && g > 2) g = 2;
  if (vpl >= 8) g = 1;
  return g;
}

Pred1Args pred1_args(const PredLaunch& p, int tok0, int nt) {
  Pred1Args a;
  a.w1_t = (const uint8_t*)p.w1_t;
  a.x = p.x;
  a.norm = p.norm;
  a.z = p.z;
  a.d = p.d;
  a.r = p.r;
  a.tok0 = tok0;
  a.nt = nt;
  return a;
}

Pred2Args pred2_args(const PredLaunch& p, int tok0, int nt) {
  Pred2Args a;
  a.w2_t = (const uint8_t*)p.w2_t;
  a.z = p.z;
  a.tau = p.tau;
  a.mask = p.mask;
  a.union_mask = p.union_mask;
  a.logits = p.logits;
  a.f = p.f;
  a.r = p.r;
  a.tok0 = tok0;
  a.nt = nt;
  a.first_pass = tok0 == 0 ? 1 : 0;
  a.hot = p.hot;
  return a;
}

template <int WT, int NT, bool CHAIN>
static void pred1_pass(const PredLaunch& p, int tok0, int nt, hipStream_t s) {
  using XT = typename std::conditional<WT == WT_F32, float, f16>::type;
  const int nvec1 = p.d * (int)sizeof(XT) / 16;
  const size_t sh1 = (size_t)NT * p.d * sizeof(XT);
  const Pred1Args a = pred1_args(p, tok0, nt);
  if (nvec1 >= 256) {
    constexpr int LPR = 64;
    const int waves = (p.r + (kWave / LPR) - 1) / (kWave / LPR);
    hipLaunchKernelGGL((k_pred1<WT, LPR, NT, CHAIN>), dim3((waves + 3) / 4), dim3(256), sh1, s, a);
  } else {
    constexpr int LPR = 16;
    const int waves = (p.r + (kWave / LPR) - 1) / (kWave / LPR);
    hipLaunchKernelGGL((k_pred1<WT, LPR, NT, CHAIN>), dim3((waves + 3) / 4), dim3(256), sh1, s, a);
  }
}

template <int WT, int NT>
static void pred1_all(const PredLaunch& p, hipStream_t s) {
  const bool chain = p.norm.r_in != nullptr;
  for (int tok0 = 0; tok0 < p.batch; tok0 += NT) {
    const int nt = (p.batch - tok0 < NT) ? (p.batch - tok0) : NT;
    if (chain)
      pred1_pass<WT, NT, true>(p, tok0, nt, s);
    else
      pred1_pass<WT, NT, false>(p, tok0, nt, s);
  }
}

template <int WT, int NT, int VPL>
static void pred2_all(const PredLaunch& p, hipStream_t s) {
  constexpr int RB = VPL <= 2 ? 8 : (VPL == 4 ? 4 : 2);
  for (int tok0 = 0; tok0 < p.batch; tok0 += NT) {
    const int nt = (p.batch - tok0 < NT) ? (p.batch - tok0) : NT;
    hipLaunchKernelGGL((k_pred2<WT, NT, VPL, RB>), dim3(p.f / 64), dim3(512), 0, s, pred2_args(p, tok0, nt));
  }
}

template <int WT, int NT>
static void pred2_vpl_all(const PredLaunch& p, hipStream_t s) {
  switch (pred2_vpl(WT, p.r)) {
    case 1: pred2_all<WT, NT, 1>(p, s); break;
    case 2: pred2_all<WT, NT, 2>(p, s); break;
    case 4: pred2_all<WT, (NT > 2 ? 2 : NT), 4>(p, s); break;
    default: pred2_all<WT, 1, 8>(p, s); break;
  }
}

template <int WT>
static void pred1_dispatch(const PredLaunch& p, hipStream_t s) {
  switch (pred_group(WT, p.d, p.r, p.batch, p.norm.r_in != nullptr)) {
    case 1: pred1_all<WT, 1>(p, s); break;
    case 2: pred1_all<WT, 2>(p, s); break;
    case 4: pred1_all<WT, 4>(p, s); break;
    default: pred1_all<WT, 8>(p, s); break;
  }
}

template <int WT>
static void pred2_dispatch(const PredLaunch& p, hipStream_t s) {
  switch (pred2_group(WT, p.r, p.batch)) {
    case 1: pred2_vpl_all<WT, 1>(p, s); break;
    case 2: pred2_vpl_all<WT, 2>(p, s); break;
    case 4: pred2_vpl_all<WT, 4>(p, s); break;
    default: pred2_vpl_all<WT, 8>(p, s); break;
  }
}

hipError_t launch_predict(const PredLaunch& p, hipStream_t s) {
  if (pred_uses_mfma(p)) {
    const hipError_t e = launch_pred1_mfma(p, s);
    return e != hipSuccess ? e : launch_pred2_mfma(p, s);
  }
  if (p.wt == WT_F32) {
    pred1_dispatch<WT_F32>(p, s);
    pred2_dispatch<WT_F32>(p, s);
  } else {
    pred1_dispatch<WT_F16>(p, s);
    pred2_dispatch<WT_F16>(p, s);
  }
  return hipGetLastError();
}

hipError_t launch_predict_stage1(const PredLaunch& p, hipStream_t s) {
  if (pred_uses_mfma(p)) return launch_pred1_mfma(p, s);
  if (p.wt == WT_F32)
    pred1_dispatch<WT_F32>(p, s);
  else
    pred1_dispatch<WT_F16>(p, s);
  return hipGetLastError();
}

hipError_t launch_predict_stage2(const PredLaunch& p, hipStream_t s) {
  if (pred_uses_mfma(p)) return launch_pred2_mfma(p, s);
  if (p.wt == WT_F32)
    pred2_dispatch<WT_F32>(p, s);
  else
    pred2_dispatch<WT_F16>(p, s);
  return hipGetLastError();
}

}  // namespace sfnn
