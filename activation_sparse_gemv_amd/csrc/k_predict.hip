// Low-rank activation predictor: z = W1^T x, logit = W2^T z, mask = logit > tau.
//
// The per-layer predictor decides which FFN neurons a token fires before the
// FFN runs (53ai.com sparsity survey, PowerInfer section 自适应稀疏预测器; the
// hexiedandong.com PowerInfer repost: a small per-layer routing module predicts
// the neurons each input activates).  The rank-r linear form is the reading
// taken here of the pages' "input, hidden, output layer" predictor.
//
// Both stages are HBM-bound GEMVs at small batch (the rank-r factors are read
// in full every token), so they are wave-per-row(s) dot products with 16-byte
// coalesced row loads.  Each wave issues its first batch of weight loads
// before the activations are staged in LDS, so the weight fetch overlaps the
// staging.  The first stage can build its own input from the previous layer's
// down-projection partials (reduce + residual + RMSNorm in the prologue), which
// removes two launches per layer from a residual stack.  The second stage fuses
// the threshold, packs 64 decisions per wavefront ballot and ORs the batch's
// words into the union mask.
#include "common.hpp"
#include "launch.hpp"

namespace sfnn {

constexpr int kChainMaxV = 16;  // float4 vectors of the residual row kept per thread

// Residual-chain prologue: for the nt tokens of this group, y = b_down +
// partials (fixed order), r = r_in + y, x = r / rms(r) into xs (and, from
// workgroup 0, r_out / y_out / x_out to global memory).  Each workgroup does
// this redundantly; the order of every sum is fixed, so every workgroup gets
// the same x.  Requires NT * d / 4 <= kChainMaxV * blockDim.x.
template <typename XT, int NT>
__device__ __forceinline__ void chain_stage(const NormIn& n, XT* xs, float (*red)[4], const void* b_down, int d,
                                            int B, int tok0, int nt) {
  const int nv = d / 4;  // float4 vectors per token row
  const int total = NT * nv;
  const int kv = (total + blockDim.x - 1) / blockDim.x;  // vectors this thread may own (<= kChainMaxV)
  const bool wg0 = blockIdx.x == 0;
  f32x4 v[kChainMaxV];
  float ss[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) ss[t] = 0.0f;
  // four vectors at a time: every load of the group (residual, bias, all
  // partials) is issued before any is used; invalid slots read token tok0's
  // row (in bounds) and are dropped by a select
#pragma unroll
  for (int k0 = 0; k0 < kChainMaxV; k0 += 4) {
    if (k0 < kv) {
      f32x4 y[4], rr[4];
      size_t off[4];
      bool val[4];
      int tk[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int e = threadIdx.x + (k0 + kk) * blockDim.x;
        const int t = e / nv, c4 = e - t * nv;
        val[kk] = e < total && t < nt;
        tk[kk] = t;
        const int cc = val[kk] ? c4 : 0;
        off[kk] = (size_t)(tok0 + (val[kk] ? t : 0)) * d + 4 * cc;
        rr[kk] = *reinterpret_cast<const f32x4*>(n.r_in + off[kk]);
        y[kk] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (b_down) {
          const XT* bd = reinterpret_cast<const XT*>(b_down) + 4 * cc;
          y[kk] = f32x4{(float)bd[0], (float)bd[1], (float)bd[2], (float)bd[3]};
        }
      }
      for (int q0 = 0; q0 < n.R; q0 += 4) {
        f32x4 p[4][4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int q = (q0 + j < n.R) ? q0 + j : q0;
            p[kk][j] = *reinterpret_cast<const f32x4*>(n.partial + (size_t)q * B * d + off[kk]);
          }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (q0 + j < n.R) y[kk] += p[kk][j];
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const f32x4 rv = rr[kk] + y[kk];
        v[k0 + kk] = val[kk] ? rv : f32x4{0.f, 0.f, 0.f, 0.f};
        float s = 0.0f;
        s = __builtin_fmaf(rv.x, rv.x, s);
        s = __builtin_fmaf(rv.y, rv.y, s);
        s = __builtin_fmaf(rv.z, rv.z, s);
        s = __builtin_fmaf(rv.w, rv.w, s);
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) ss[tt] += (val[kk] && tt == tk[kk]) ? s : 0.0f;
        if (wg0 && val[kk]) {
          if (n.r_out) *reinterpret_cast<f32x4*>(n.r_out + off[kk]) = rv;
          if (n.y_out) *reinterpret_cast<f32x4*>(n.y_out + off[kk]) = y[kk];
        }
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) v[k0 + kk] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float s = group_sum<kWave>(ss[t]);
    if (lane == 0) red[t][wave] = s;
  }
  __syncthreads();
  float inv[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float tot = ((red[t][0] + red[t][1]) + red[t][2]) + red[t][3];
    inv[t] = 1.0f / __builtin_sqrtf(tot / (float)d + n.eps);
  }
#pragma unroll
  for (int k = 0; k < kChainMaxV; ++k) {
    const int e = threadIdx.x + k * blockDim.x;
    if (e < total) {
      const int t = e / nv, c4 = e - t * nv;
      float sc = 0.0f;
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) sc = (tt == t) ? inv[tt] : sc;
      const f32x4 o = v[k] * sc;  // tokens >= nt stage zeros
      XT* dst = xs + (size_t)t * d + 4 * c4;
      dst[0] = (XT)o.x;
      dst[1] = (XT)o.y;
      dst[2] = (XT)o.z;
      dst[3] = (XT)o.w;
      if (wg0 && t < nt) {
        XT* xo = reinterpret_cast<XT*>(n.x_out) + (size_t)(tok0 + t) * d + 4 * c4;
        xo[0] = dst[0];
        xo[1] = dst[1];
        xo[2] = dst[2];
        xo[3] = dst[3];
      }
    }
  }
}

// Stage 1: z[tok][j] = sum_k w1_t[j][k] x[tok][k] for tokens [tok0, tok0+nt).
template <int WT, int LPR, int NT, bool CHAIN>
__global__ __launch_bounds__(256) void k_pred1(const uint8_t* __restrict__ w1_t, const void* __restrict__ x,
                                               NormIn nrm, float* __restrict__ z, int d, int r, int B, int tok0,
                                               int nt) {
  using XT = typename std::conditional<WT == WT_F32, float, f16>::type;
  constexpr int UB = 8;
  constexpr int RPW = kWave / LPR;  // rows per wave per step
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ float red[NT][4];
  XT* xs = reinterpret_cast<XT*>(smem);

  const int lane = threadIdx.x & (kWave - 1);
  const int li = lane % LPR;
  const int gw = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int GW = gridDim.x * (blockDim.x / kWave);
  const int row_bytes = d * (int)sizeof(XT);
  const int nvec = row_bytes / 16;

  // first batch of this lane group's first row, in flight during the staging
  RowLoads<WT, LPR, UB> L;
  const int j0 = gw * RPW + lane / LPR;
  const bool pre = j0 < r && li < nvec;
  if (pre) L.issue(w1_t + (size_t)j0 * row_bytes, nullptr, nvec, li);

  if constexpr (CHAIN)
    chain_stage<XT, NT>(nrm, xs, red, nrm.b_down, d, B, tok0, nt);
  else
    stage_rows<XT, false>(xs, reinterpret_cast<const XT*>(x), d, tok0, nt, NT);
  __syncthreads();

  for (int base = gw * RPW; base < r; base += GW * RPW) {
    const int j = base + lane / LPR;
    float acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = 0.0f;
    if (j < r)
      row_dot<WT, LPR, UB, NT, XT>(L, pre && base == gw * RPW, w1_t + (size_t)j * row_bytes, nullptr, nvec, li, xs,
                                   d, acc);
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = group_sum<LPR>(acc[t]);
    if (li == 0 && j < r) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
        if (t < nt) z[(size_t)(tok0 + t) * r + j] = acc[t];
    }
  }
}

// Stage 2: one workgroup = 64 neurons = one mask word per token.  8 waves,
// each wave 8 rows at a time with 8 lanes per row.  Writes the mask words of
// tokens [tok0, tok0+nt) and ORs them into union_mask (first pass: stores).
template <int WT, int NT>
__global__ __launch_bounds__(512) void k_pred2(const uint8_t* __restrict__ w2_t, const float* __restrict__ z,
                                               const float* __restrict__ tau, uint64_t* __restrict__ mask,
                                               uint64_t* __restrict__ union_mask, float* __restrict__ logits, int f,
                                               int r, int tok0, int nt, int first_pass) {
  constexpr int LPR = 8, UB = 16;
  extern __shared__ __align__(16) unsigned char smem[];
  float* zs = reinterpret_cast<float*>(smem);
  __shared__ float lg[NT][64];
  __shared__ unsigned long long wsh[NT];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int li = lane % LPR;
  const int local = wave * (kWave / LPR) + lane / LPR;  // 0..63
  const int i = blockIdx.x * 64 + local;
  const int row_bytes = r * (WT == WT_F32 ? 4 : 2);
  const int nvec = row_bytes / 16;

  RowLoads<WT, LPR, UB> L;
  const bool pre = li < nvec;
  if (pre) L.issue(w2_t + (size_t)i * row_bytes, nullptr, nvec, li);
  const float tv = tau[blockIdx.x * 64 + lane];

  stage_rows<float, false>(zs, z, r, tok0, nt, NT);
  __syncthreads();

  float acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = 0.0f;
  row_dot<WT, LPR, UB, NT, float>(L, pre, w2_t + (size_t)i * row_bytes, nullptr, nvec, li, zs, r, acc);
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = group_sum<LPR>(acc[t]);
  if (li == 0) {
#pragma unroll
    for (int t = 0; t < NT; ++t) lg[t][local] = acc[t];
  }
  __syncthreads();

  if (wave < nt) {
    const int tok = tok0 + wave;
    const float v = lg[wave][lane];
    const bool on = v > tv;
    const unsigned long long word = __ballot(on);
    if (lane == 0) {
      mask[(size_t)tok * (f / 64) + blockIdx.x] = (uint64_t)word;
      wsh[wave] = word;
    }
    if (logits) logits[(size_t)tok * f + blockIdx.x * 64 + lane] = v;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t u = first_pass ? 0ull : union_mask[blockIdx.x];
    for (int t = 0; t < nt; ++t) u |= wsh[t];
    union_mask[blockIdx.x] = u;
  }
}

static int pow2_floor(int v) {
  int p = 1;
  while (p * 2 <= v) p *= 2;
  return p;
}

int pred_group(int wt, int d, int r, int batch, bool chain) {
  const int xb = (wt == WT_F32) ? 4 : 2;
  int per_tok = d * xb;
  if (r * 4 > per_tok) per_tok = r * 4;
  int cap = kStageBytes / per_tok;
  if (chain) {
    const int cap2 = kChainMaxV * 256 * 4 / d;  // residual rows held in registers
    if (cap2 < cap) cap = cap2;
  }
  if (cap < 1) cap = 1;
  if (cap > kMaxNT) cap = kMaxNT;
  cap = pow2_floor(cap);
  int nt = 1;
  while (nt < batch && nt < cap) nt *= 2;
  return nt;
}

template <int WT, int NT, bool CHAIN>
static void pred_pass(const PredLaunch& p, int tok0, int nt, hipStream_t s) {
  using XT = typename std::conditional<WT == WT_F32, float, f16>::type;
  const int nvec1 = p.d * (int)sizeof(XT) / 16;
  const size_t sh1 = (size_t)NT * p.d * sizeof(XT);
  const void* x = p.x;
  if (nvec1 >= 256) {
    constexpr int LPR = 64;
    const int waves = (p.r + (kWave / LPR) - 1) / (kWave / LPR);
    hipLaunchKernelGGL((k_pred1<WT, LPR, NT, CHAIN>), dim3((waves + 3) / 4), dim3(256), sh1, s,
                       (const uint8_t*)p.w1_t, x, p.norm, p.z, p.d, p.r, p.batch, tok0, nt);
  } else {
    constexpr int LPR = 16;
    const int waves = (p.r + (kWave / LPR) - 1) / (kWave / LPR);
    hipLaunchKernelGGL((k_pred1<WT, LPR, NT, CHAIN>), dim3((waves + 3) / 4), dim3(256), sh1, s,
                       (const uint8_t*)p.w1_t, x, p.norm, p.z, p.d, p.r, p.batch, tok0, nt);
  }
}

template <int WT, int NT>
static void pred2_pass(const PredLaunch& p, int tok0, int nt, hipStream_t s) {
  const size_t sh2 = (size_t)NT * p.r * sizeof(float);
  hipLaunchKernelGGL((k_pred2<WT, NT>), dim3(p.f / 64), dim3(512), sh2, s, (const uint8_t*)p.w2_t, p.z, p.tau,
                     p.mask, p.union_mask, p.logits, p.f, p.r, tok0, nt, tok0 == 0 ? 1 : 0);
}

template <int WT, int NT>
static void pred_all_nt(const PredLaunch& p, hipStream_t s) {
  const bool chain = p.norm.r_in != nullptr;
  for (int tok0 = 0; tok0 < p.batch; tok0 += NT) {
    const int nt = (p.batch - tok0 < NT) ? (p.batch - tok0) : NT;
    if (chain)
      pred_pass<WT, NT, true>(p, tok0, nt, s);
    else
      pred_pass<WT, NT, false>(p, tok0, nt, s);
  }
  for (int tok0 = 0; tok0 < p.batch; tok0 += NT) {
    const int nt = (p.batch - tok0 < NT) ? (p.batch - tok0) : NT;
    pred2_pass<WT, NT>(p, tok0, nt, s);
  }
}

template <int WT>
static void pred_all(const PredLaunch& p, hipStream_t s) {
  switch (pred_group(WT, p.d, p.r, p.batch, p.norm.r_in != nullptr)) {
    case 1: pred_all_nt<WT, 1>(p, s); break;
    case 2: pred_all_nt<WT, 2>(p, s); break;
    case 4: pred_all_nt<WT, 4>(p, s); break;
    default: pred_all_nt<WT, 8>(p, s); break;
  }
}

hipError_t launch_predict(const PredLaunch& p, hipStream_t s) {
  if (p.wt == WT_F32)
    pred_all<WT_F32>(p, s);
  else
    pred_all<WT_F16>(p, s);
  return hipGetLastError();
}

}  // namespace sfnn
