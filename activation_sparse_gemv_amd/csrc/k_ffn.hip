// FFN launches: k_ffn (the one-launch gathered FFN) and k_sum (fixed-order
// sum of the workgroups' partials).  The workgroup bodies live in
// ffn_body.hpp.
#include "ffn_launch.hpp"

#ifndef SFNN_FFN_WGS
#define SFNN_FFN_WGS 256  // FFN workgroups (raised when d_ff / kMaxPer needs more)
#endif

namespace sfnn {

__global__ __launch_bounds__(512) void k_sum(SumArgs a) { sum_body(a, blockIdx.x, gridDim.x); }

// The same sum when there are few partial rows (the matrix-core paths write 8
// or 16 per token): 4 consecutive elements per thread, the rows added one
// after another from zero, then the bias, then the residual, exactly the
// order k_sum takes with at most 32 rows, so both give the same bits.
__global__ __launch_bounds__(256) void k_sum_wide(SumArgs a) {
  const int n = a.B * a.d;
  const int e = (blockIdx.x * 256 + threadIdx.x) * 4;  // d is a multiple of 128: 4 elements never straddle
  if (e >= n) return;
  float t[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 8
  for (int g = 0; g < a.G; ++g) {
    const f32x4 p = *reinterpret_cast<const f32x4*>(a.partial + (size_t)g * n + e);
    t[0] += p.x;
    t[1] += p.y;
    t[2] += p.z;
    t[3] += p.w;
  }
  const int c = e % a.d;
  float v[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float b = 0.0f;
    if (a.b_down) b = (a.xtype == WT_F32) ? load_as_float<float>(a.b_down, c + k) : load_as_float<f16>(a.b_down, c + k);
    v[k] = b + t[k];
  }
  if (a.y) *reinterpret_cast<f32x4*>(a.y + e) = f32x4{v[0], v[1], v[2], v[3]};
  if (a.r_in) {
    const f32x4 r = *reinterpret_cast<const f32x4*>(a.r_in + e);
    *reinterpret_cast<f32x4*>(a.r_out + e) = f32x4{r.x + v[0], r.y + v[1], r.z + v[2], r.w + v[3]};
  }
}

// Threads own CPT columns each for the down projection (at most 512
// threads); the token group is bounded by the staged activations (LDS) and by
// 64 accumulators per thread.
FfnShape ffn_shape(int wt, int d, int batch) {
  FfnShape s;
  s.cpt = d <= 4096 ? 8 : (d <= 8192 ? 16 : 32);
  const int need = d / s.cpt;
  s.nth = need <= 256 ? 256 : 512;
  const int xb = (wt == WT_F32) ? 4 : 2;
  int cap = kStageBytes / (d * xb);
  const int acc_cap = 64 / s.cpt;
  if (cap > acc_cap) cap = acc_cap;
  if (cap < 1) cap = 1;
  if (cap > kMaxNT) cap = kMaxNT;
  int c2 = 1;
  while (c2 * 2 <= cap) c2 *= 2;
  s.nt = 1;
  while (s.nt < batch && s.nt < c2) s.nt *= 2;
  return s;
}

int ffn_groups(int d, int f) {
  (void)d;
  int G = SFNN_FFN_WGS;
  const int need = (f + kMaxPer - 1) / kMaxPer;  // every slot must fit some workgroup's LDS list
  if (G < need) G = need;
  if (G > f / 4) G = f / 4 > need ? f / 4 : need;
  return G;
}

FfnArgs ffn_args(const FfnLaunch& p, int tok0, int nt, bool first) {
  FfnArgs a;
  a.w_up = (const uint8_t*)p.w_up;
  a.w_gate = (const uint8_t*)p.w_gate;
  a.w_down_t = (const uint8_t*)p.w_down_t;
  a.s_up = (const f16*)p.s_up;
  a.s_gate = (const f16*)p.s_gate;
  a.s_down_t = (const f16*)p.s_down_t;
  a.b_up = p.b_up;
  a.b_gate = p.b_gate;
  a.x = p.x;
  a.ids = p.ids;
  a.count = p.count;
  a.union_mask = p.union_mask;
  a.ids_out = p.ids_out;
  a.count_out = p.count_out;
  a.mask = p.mask;
  a.partial = p.partial;
  a.r_in = nullptr;
  a.x_out = nullptr;
  a.eps = 0.0f;
  a.w1_t = nullptr;
  a.z = nullptr;
  a.r = 0;
  a.d = p.d;
  a.f = p.f;
  a.B = p.batch;
  a.tok0 = tok0;
  a.nt = nt;
  a.write_ids = (p.src == SRC_UNION && first) ? 1 : 0;
  return a;
}

SumArgs sum_args(const FfnLaunch& p) {
  SumArgs a;
  a.partial = p.partial;
  a.G = ffn_uses_mfma(p) ? mfma_groups(p.d, p.groups) : p.groups;
  a.B = p.batch;
  a.d = p.d;
  a.xtype = p.wt == WT_F32 ? WT_F32 : WT_F16;
  a.b_down = p.b_down;
  a.y = p.y;
  a.r_in = p.r_in;
  a.r_out = p.r_out;
  return a;
}

int sum_groups(int batch, int d) { return (batch * d + kSumEPW - 1) / kSumEPW; }  // 512-thread workgroups

hipError_t launch_sum(const FfnLaunch& p, hipStream_t s) {
  const SumArgs a = sum_args(p);
  if (a.G <= 32) {
    const int n4 = (p.batch * p.d) / 4;
    hipLaunchKernelGGL(k_sum_wide, dim3((n4 + 255) / 256), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL(k_sum, dim3(sum_groups(p.batch, p.d)), dim3(512), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_ffn(const FfnLaunch& p, hipStream_t s) {
  if (ffn_uses_mfma(p)) return launch_ffn_mfma(p, s);
  if (p.wt == WT_F32)
    ffn_run_f32(p, s);
  else if (p.wt == WT_F16)
    ffn_run_f16(p, s);
  else
    ffn_run_i4(p, s);
  return hipGetLastError();
}

}  // namespace sfnn
