// Host side of the per-row FFN (k_up + k_down, bodies in ffn_body.hpp and
// down_body.hpp) and k_sum / k_sum_wide, the fixed-order sums of the
// matrix-core paths' partial rows.
#include "ffn_launch.hpp"

#ifndef SFNN_FFN_WGS
#define SFNN_FFN_WGS 256  // up-projection workgroups (raised when d_ff / kMaxPer needs more)
#endif

namespace sfnn {

__global__ __launch_bounds__(512) void k_sum(SumArgs a) { sum_body(a, blockIdx.x, gridDim.x); }

// The same sum when there are few partial rows (the matrix-core paths write 8
// to 32 per token, the per-row down projection's row groups up to 16): 4
// consecutive elements per thread, the rows added one after another from
// zero, then the bias, then the residual, exactly the order k_sum takes with
// at most 32 rows, so both give the same bits.  64-thread workgroups, so a
// single token's row spreads over many CUs; the bias and residual loads go
// out with the partial rows.
constexpr int kSumWideThreads = 64;
__global__ __launch_bounds__(kSumWideThreads) void k_sum_wide(SumArgs a) {
  const int n = a.B * a.d;
  const int e = (blockIdx.x * kSumWideThreads + threadIdx.x) * 4;  // d is a multiple of 128: 4 elements never straddle
  if (e >= n) return;
  const int c = e % a.d;
  float b[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (a.b_down) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      b[k] = (a.xtype == WT_F32) ? load_as_float<float>(a.b_down, c + k) : load_as_float<f16>(a.b_down, c + k);
  }
  f32x4 r = {0.0f, 0.0f, 0.0f, 0.0f};
  if (a.r_in) r = *reinterpret_cast<const f32x4*>(a.r_in + e);
  float t[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 8
  for (int g = 0; g < a.G; ++g) {
    const f32x4 p = *reinterpret_cast<const f32x4*>(a.partial + (size_t)g * n + e);
    t[0] += p.x;
    t[1] += p.y;
    t[2] += p.z;
    t[3] += p.w;
  }
  float v[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) v[k] = b[k] + t[k];
  if (a.y) *reinterpret_cast<f32x4*>(a.y + e) = f32x4{v[0], v[1], v[2], v[3]};
  if (a.r_in) *reinterpret_cast<f32x4*>(a.r_out + e) = f32x4{r.x + v[0], r.y + v[1], r.z + v[2], r.w + v[3]};
}

// Up projection: 512 threads; the token group is bounded by the staged
// activations (LDS).  rv: float4 vectors per thread per token that hold a
// residual row in the look-ahead prologue (d_model <= 4 rv 512).
FfnShape ffn_shape(int wt, int d, int batch) {
  FfnShape s;
  s.rv = d <= 4096 ? 2 : (d <= 8192 ? 4 : 8);
  s.nth = 512;
  const int xb = (wt == WT_F32) ? 4 : 2;
  int cap = kStageBytes / (d * xb);
  if (cap < 1) cap = 1;
  if (cap > kMaxNT) cap = kMaxNT;
  int c2 = 1;
  while (c2 * 2 <= cap) c2 *= 2;
  s.nt = 1;
  while (s.nt < batch && s.nt < c2) s.nt *= 2;
  return s;
}

// Down projection: with items > 0, tiles of whole 128-byte lines (8 lanes of
// 16 bytes) where the row is a multiple of them, else 64 or 32 bytes, and as
// many row groups as bring the work items near `items` (at most
// kDownMaxGroups); with items == 0, one row group; tokens per pass
// bounded by 64 accumulators per lane (fp32: 4, fp16: 8, INT4: 32 columns per
// lane).
DownShape down_shape(int wt, int d, int batch, int items) {
  DownShape s;
  const int vecs = down_row_bytes(wt, d) / 16;  // 16-byte vectors per row (a multiple of 4)
  if (items > 0) {
    s.lpr = vecs % 8 == 0 ? 8 : (vecs % 4 == 0 ? 4 : 2);
    s.tiles = vecs / s.lpr;
    s.rg = (items + s.tiles / 2) / s.tiles;
    if (s.rg < 1) s.rg = 1;
    if (s.rg > kDownMaxGroups) s.rg = kDownMaxGroups;
  } else {
    // no row groups: the narrowest tile with at most 256 tiles per row
    s.lpr = 1;
    while (s.lpr < 8 && vecs / s.lpr > 256 && (vecs % (2 * s.lpr)) == 0) s.lpr *= 2;
    s.tiles = vecs / s.lpr;
    s.rg = 1;
  }
  const int cpl = wt == WT_F32 ? 4 : (wt == WT_F16 ? 8 : 32);
  int cap = 64 / cpl;
  if (cap > kMaxNT) cap = kMaxNT;
  s.nt = 1;
  while (s.nt < batch && s.nt < cap) s.nt *= 2;
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
  a.hout = p.hrow;
  a.hstride = p.f;
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

DownArgs ffn_down_args(const FfnLaunch& p) {
  DownArgs a;
  a.w = (const uint8_t*)p.w_down_t;
  a.s = (const f16*)p.s_down_t;
  if (p.src == SRC_UNION) {
    a.ids = p.ids_out;
    a.count = p.count_out;
  } else if (p.src == SRC_IDS) {
    a.ids = p.ids;
    a.count = p.count;
  } else {
    a.ids = nullptr;
    a.count = nullptr;
  }
  a.n_slots = p.f;
  a.n_rows = p.f;
  a.co = p.hrow;
  a.co_stride = p.f;
  a.bias = p.b_down;
  a.bias_f32 = p.wt == WT_F32 ? 1 : 0;
  a.y = p.y;
  a.r_in = p.r_in;
  a.r_out = p.r_out;
  a.d = p.d;
  a.tok0 = 0;
  a.nt = p.batch;
  a.rg = 1;
  a.part = p.partial;
  a.batch = p.batch;
  return a;
}

// The row groups' partial rows of a down projection added into y / the
// residual row (fixed order), with the bias.
hipError_t launch_down_sum(const DownArgs& d, hipStream_t s) {
  SumArgs a;
  a.partial = d.part;
  a.G = d.rg;
  a.B = d.batch;
  a.d = d.d;
  a.xtype = d.bias_f32 ? WT_F32 : WT_F16;
  a.b_down = d.bias;
  a.y = d.y;
  a.r_in = d.r_in;
  a.r_out = d.r_out;
  return launch_sum_args(a, s);
}

SumArgs sum_args(const FfnLaunch& p, int rows) {
  SumArgs a;
  a.partial = p.partial;
  a.G = rows;
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

hipError_t launch_sum_args(const SumArgs& a, hipStream_t s) {
  if (a.G <= 32) {
    const int n4 = (a.B * a.d) / 4;
    hipLaunchKernelGGL(k_sum_wide, dim3((n4 + kSumWideThreads - 1) / kSumWideThreads), dim3(kSumWideThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL(k_sum, dim3(sum_groups(a.B, a.d)), dim3(512), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_sum(const FfnLaunch& p, int rows, hipStream_t s) { return launch_sum_args(sum_args(p, rows), s); }

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
