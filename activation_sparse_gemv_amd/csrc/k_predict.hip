// Low-rank activation predictor: z = W1^T x, logit = W2^T z, mask = logit > tau.
//
// The per-layer predictor decides which FFN neurons a token fires before the
// FFN runs (53ai.com sparsity survey, PowerInfer section 自适应稀疏预测器; the
// hexiedandong.com PowerInfer repost: a small per-layer routing module predicts
// the neurons each input activates).  The rank-r linear form is the reading
// taken here of the pages' "input, hidden, output layer" predictor.
//
// Both stages are HBM-bound GEMVs at small batch (the rank-r factors are read
// in full every token).  Activation loads are issued first and weight loads
// right behind them, so the activations arrive while the weights stream in.
//   k_pred1: one wavefront per row of W1^T, x staged in LDS.  In a residual
//            stack the prologue builds x = r / rms(r) from the residual row.
//   k_pred2: a workgroup owns 64 neurons (one mask word per token); each
//            wavefront takes 8 rows of W2^T with all 64 lanes on every row and
//            z held in registers, so z is read once per lane instead of once
//            per row; the 8 row sums are formed by one multi-row butterfly.
//            The threshold is fused, 64 decisions are packed per __ballot and
//            the batch's words are ORed into the union mask.
#include "common.hpp"
#include "launch.hpp"

namespace sfnn {

constexpr int kChainMaxV = 16;  // float4 vectors of the residual rows kept per thread

// Residual-chain prologue, issue half: this thread's float4 vectors of the
// nt residual rows (zeros past nt).  Requires NT * d / 4 <= kChainMaxV * blockDim.x.
__device__ __forceinline__ void chain_issue(const NormIn& n, f32x4 (&v)[kChainMaxV], int d, int tok0, int nt,
                                            int NT) {
  const int nv = d / 4;
  const int total = NT * nv;
#pragma unroll
  for (int k = 0; k < kChainMaxV; ++k) {
    const int e = threadIdx.x + k * blockDim.x;
    const int t = e / nv;
    const bool ok = e < total && t < nt;
    const size_t off = ok ? (size_t)(tok0 + t) * d + 4 * (e - t * nv) : (size_t)tok0 * d;
    const f32x4 r = *reinterpret_cast<const f32x4*>(n.r_in + off);
    v[k] = ok ? r : f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// Finish half: x = r / sqrt(mean(r^2) + eps) rounded to XT into xs (and, from
// workgroup 0, into x_out).  Every workgroup sums in the same fixed order, so
// all get the same x.
template <typename XT, int NT>
__device__ __forceinline__ void chain_finish(const NormIn& n, const f32x4 (&v)[kChainMaxV], XT* xs,
                                             float (*red)[16], int d, int tok0, int nt) {
  const int nv = d / 4;
  const int total = NT * nv;
  const int nw = blockDim.x / kWave;
  float ss[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) ss[t] = 0.0f;
#pragma unroll
  for (int k = 0; k < kChainMaxV; ++k) {
    const int e = threadIdx.x + k * blockDim.x;
    const int t = e / nv;
    float s = 0.0f;
    s = __builtin_fmaf(v[k].x, v[k].x, s);
    s = __builtin_fmaf(v[k].y, v[k].y, s);
    s = __builtin_fmaf(v[k].z, v[k].z, s);
    s = __builtin_fmaf(v[k].w, v[k].w, s);
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) ss[tt] += (e < total && tt == t) ? s : 0.0f;
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
    float tot = 0.0f;
    for (int w = 0; w < nw; ++w) tot += red[t][w];
    inv[t] = 1.0f / __builtin_sqrtf(tot / (float)d + n.eps);
  }
  const bool wg0 = blockIdx.x == 0;
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
                                               NormIn nrm, float* __restrict__ z, int d, int r, int tok0, int nt) {
  using XT = typename std::conditional<WT == WT_F32, float, f16>::type;
  constexpr int UB = 8;
  constexpr int RPW = kWave / LPR;  // rows per wave per step
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ float red[NT][16];
  XT* xs = reinterpret_cast<XT*>(smem);

  const int lane = threadIdx.x & (kWave - 1);
  const int li = lane % LPR;
  const int gw = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int GW = gridDim.x * (blockDim.x / kWave);
  const int row_bytes = d * (int)sizeof(XT);
  const int nvec = row_bytes / 16;

  // activations first, then this lane group's first batch of its first row
  f32x4 rv[kChainMaxV];
  StageSplit<XT, false, 2> stage;
  if constexpr (CHAIN)
    chain_issue(nrm, rv, d, tok0, nt, NT);
  else
    stage.issue(reinterpret_cast<const XT*>(x), d, tok0, nt, NT);
  RowLoads<WT, LPR, UB> L;
  const int j0 = gw * RPW + lane / LPR;
  const bool pre = j0 < r && li < nvec;
  if (pre) L.issue(w1_t + (size_t)j0 * row_bytes, nullptr, nvec, li);
  if constexpr (CHAIN)
    chain_finish<XT, NT>(nrm, rv, xs, red, d, tok0, nt);
  else
    stage.commit(xs, reinterpret_cast<const XT*>(x), d, tok0, nt, NT);
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

// Multi-row butterfly: v[k] holds this lane's partial sum of row k (k < RB).
// Returns, in lane L, the 64-lane total of row (L >> (6 - log2 RB)) & (RB-1).
// Each stage halves the rows a lane carries: the lane keeps one half and
// receives its partner's partial of that half; then the lanes that still
// share a row add across the remaining lane bits.
template <int RB>
__device__ __forceinline__ float rows_sum(float (&v)[RB]) {
  const int lane = threadIdx.x & (kWave - 1);
  int m = kWave / 2;
#pragma unroll
  for (int c = RB; c > 1; c >>= 1) {
    const bool hi = (lane & m) != 0;
#pragma unroll
    for (int k = 0; k < c / 2; ++k) {
      const float send = hi ? v[k] : v[k + c / 2];
      const float keep = hi ? v[k + c / 2] : v[k];
      v[k] = keep + __shfl_xor(send, m, kWave);
    }
    m >>= 1;
  }
  float s = v[0];
#pragma unroll
  for (int mm = kWave / (2 * RB); mm >= 1; mm >>= 1) s += __shfl_xor(s, mm, kWave);
  return s;
}

template <int RB>
constexpr int log2c() { return RB == 1 ? 0 : 1 + log2c<RB / 2>(); }

// Stage 2: workgroup = 64 neurons = one mask word per token; 8 waves of 8
// rows; VPL 16-byte vectors per lane per row; RB rows in flight per wave.
template <int WT, int NT, int VPL, int RB>
__global__ __launch_bounds__(512) void k_pred2(const uint8_t* __restrict__ w2_t, const float* __restrict__ z,
                                               const float* __restrict__ tau, uint64_t* __restrict__ mask,
                                               uint64_t* __restrict__ union_mask, float* __restrict__ logits, int f,
                                               int r, int tok0, int nt, int first_pass) {
  constexpr int E = vec_elems<WT>();  // 4 (fp32) or 8 (fp16) weights per vector
  __shared__ float lg[NT][64];
  __shared__ unsigned long long wsh[NT];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int row_bytes = r * (WT == WT_F32 ? 4 : 2);
  const int nvec = row_bytes / 16;

  // z elements of this lane's vectors (lane + 64u), straight to registers.
  // Out-of-range vectors and tokens read an in-bounds z element and are
  // cancelled later (zero weights / unused token), so nothing here waits for
  // the loads and the weight loads below go out right behind them.
  f32x4 zf[NT][VPL][E / 4];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int u = 0; u < VPL; ++u) {
      const int v = lane + kWave * u;
      const bool ok = v < nvec && t < nt;
      const float* src = z + (size_t)(tok0 + (t < nt ? t : 0)) * r + (size_t)(ok ? v : 0) * E;
#pragma unroll
      for (int q = 0; q < E / 4; ++q) zf[t][u][q] = *reinterpret_cast<const f32x4*>(src + 4 * q);
    }
  const float tv = tau[blockIdx.x * 64 + lane];

#pragma unroll
  for (int rb0 = 0; rb0 < 8; rb0 += RB) {
    u32x4 w[RB][VPL];
#pragma unroll
    for (int k = 0; k < RB; ++k) {
      const int i = blockIdx.x * 64 + wave * 8 + rb0 + k;
#pragma unroll
      for (int u = 0; u < VPL; ++u) {
        const int v = lane + kWave * u;
        w[k][u] = ld16_stream(w2_t + (size_t)i * row_bytes + 16 * (size_t)(v < nvec ? v : 0));
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // the rows' loads all issue before any math
    constexpr int SH = 6 - log2c<RB>();
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float acc[RB];
#pragma unroll
      for (int k = 0; k < RB; ++k) {
        float s = 0.0f;
#pragma unroll
        for (int u = 0; u < VPL; ++u) {
          const u32x4 wv = (lane + kWave * u < nvec) ? w[k][u] : u32x4{0u, 0u, 0u, 0u};
          const float* zz = reinterpret_cast<const float*>(&zf[t][u][0]);
          if constexpr (WT == WT_F32) {
            s = __builtin_fmaf(bitcast<float>(wv.x), zz[0], s);
            s = __builtin_fmaf(bitcast<float>(wv.y), zz[1], s);
            s = __builtin_fmaf(bitcast<float>(wv.z), zz[2], s);
            s = __builtin_fmaf(bitcast<float>(wv.w), zz[3], s);
          } else {
            const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
              const f16x2 h = bitcast<f16x2>(ww[m]);
              s = __builtin_fmaf((float)h.x, zz[2 * m], s);
              s = __builtin_fmaf((float)h.y, zz[2 * m + 1], s);
            }
          }
        }
        acc[k] = s;
      }
      const float tot = rows_sum<RB>(acc);
      if ((lane & ((1 << SH) - 1)) == 0) lg[t][wave * 8 + rb0 + ((lane >> SH) & (RB - 1))] = tot;
    }
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

static int group_for(int batch, int cap) {
  if (cap < 1) cap = 1;
  if (cap > kMaxNT) cap = kMaxNT;
  cap = pow2_floor(cap);
  int nt = 1;
  while (nt < batch && nt < cap) nt *= 2;
  return nt;
}

// Token group of stage 1: staged x in LDS, and in a residual stack the
// residual rows held in registers.
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
static int pred2_vpl(int wt, int r) {
  const int nvec = r * (wt == WT_F32 ? 4 : 2) / 16;
  int vpl = 1;
  while (vpl * kWave < nvec) vpl *= 2;
  return vpl;
}

// Token group of stage 2: z in registers, NT * VPL * E <= 64 floats.
static int pred2_group(int wt, int r, int batch) {
  const int E = (wt == WT_F32) ? 4 : 8;
  return group_for(batch, 64 / (pred2_vpl(wt, r) * E));
}

template <int WT, int NT, bool CHAIN>
static void pred1_pass(const PredLaunch& p, int tok0, int nt, hipStream_t s) {
  using XT = typename std::conditional<WT == WT_F32, float, f16>::type;
  const int nvec1 = p.d * (int)sizeof(XT) / 16;
  const size_t sh1 = (size_t)NT * p.d * sizeof(XT);
  if (nvec1 >= 256) {
    constexpr int LPR = 64;
    const int waves = (p.r + (kWave / LPR) - 1) / (kWave / LPR);
    hipLaunchKernelGGL((k_pred1<WT, LPR, NT, CHAIN>), dim3((waves + 3) / 4), dim3(256), sh1, s,
                       (const uint8_t*)p.w1_t, p.x, p.norm, p.z, p.d, p.r, tok0, nt);
  } else {
    constexpr int LPR = 16;
    const int waves = (p.r + (kWave / LPR) - 1) / (kWave / LPR);
    hipLaunchKernelGGL((k_pred1<WT, LPR, NT, CHAIN>), dim3((waves + 3) / 4), dim3(256), sh1, s,
                       (const uint8_t*)p.w1_t, p.x, p.norm, p.z, p.d, p.r, tok0, nt);
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
    hipLaunchKernelGGL((k_pred2<WT, NT, VPL, RB>), dim3(p.f / 64), dim3(512), 0, s, (const uint8_t*)p.w2_t, p.z,
                       p.tau, p.mask, p.union_mask, p.logits, p.f, p.r, tok0, nt, tok0 == 0 ? 1 : 0);
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
static void pred_all(const PredLaunch& p, hipStream_t s) {
  switch (pred_group(WT, p.d, p.r, p.batch, p.norm.r_in != nullptr)) {
    case 1: pred1_all<WT, 1>(p, s); break;
    case 2: pred1_all<WT, 2>(p, s); break;
    case 4: pred1_all<WT, 4>(p, s); break;
    default: pred1_all<WT, 8>(p, s); break;
  }
  switch (pred2_group(WT, p.r, p.batch)) {
    case 1: pred2_vpl_all<WT, 1>(p, s); break;
    case 2: pred2_vpl_all<WT, 2>(p, s); break;
    case 4: pred2_vpl_all<WT, 4>(p, s); break;
    default: pred2_vpl_all<WT, 8>(p, s); break;
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
