// Low-rank activation predictor: z = W1^T x, logit = W2^T z, mask = logit > tau.
//
// The per-layer predictor decides which FFN neurons a token fires before the
// FFN runs (53ai.com sparsity survey, PowerInfer section 自适应稀疏预测器; the
// hexiedandong.com PowerInfer repost: a small per-layer routing module predicts
// the neurons each input activates).  The rank-r linear form is the reading
// taken here of the pages' "input, hidden, output layer" predictor.
//
// Both stages are HBM-bound GEMVs at small batch (the rank-r factors are read
// in full every token), so they are plain wave-per-row(s) dot products with
// 16-byte coalesced row loads and the activations staged in LDS.  The second
// stage fuses the threshold and packs 64 decisions per wavefront ballot.
#include "common.hpp"
#include "launch.hpp"

namespace sfnn {

// Stage 1: z[tok][j] = sum_k w1_t[j][k] x[tok][k] for tokens [tok0, tok0+nt).
template <int WT, int LPR, int NT>
__global__ __launch_bounds__(256) void k_pred1(const uint8_t* __restrict__ w1_t, const void* __restrict__ x,
                                               float* __restrict__ z, int d, int r, int tok0, int nt) {
  using XT = typename std::conditional<WT == WT_F32, float, f16>::type;
  extern __shared__ __align__(16) unsigned char smem[];
  XT* xs = reinterpret_cast<XT*>(smem);
  stage_rows<XT, false>(xs, reinterpret_cast<const XT*>(x), d, tok0, nt, NT);
  __syncthreads();

  constexpr int RPW = kWave / LPR;  // rows per wave per step
  const int lane = threadIdx.x & (kWave - 1);
  const int li = lane % LPR;
  const int gw = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int GW = gridDim.x * (blockDim.x / kWave);
  const int row_bytes = d * (WT == WT_F32 ? 4 : 2);
  const int nvec = row_bytes / 16;

  for (int base = gw * RPW; base < r; base += GW * RPW) {
    const int j = base + lane / LPR;
    float acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = 0.0f;
    if (j < r) row_partial<WT, LPR, NT, 8, XT>(w1_t + (size_t)j * row_bytes, nullptr, nvec, li, xs, d, acc);
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
// each wave 8 rows at a time with 8 lanes per row.
template <int WT, int NT>
__global__ __launch_bounds__(512) void k_pred2(const uint8_t* __restrict__ w2_t, const float* __restrict__ z,
                                               const float* __restrict__ tau, uint64_t* __restrict__ mask,
                                               float* __restrict__ logits, int f, int r, int tok0, int nt) {
  constexpr int LPR = 8;
  extern __shared__ __align__(16) unsigned char smem[];
  float* zs = reinterpret_cast<float*>(smem);
  __shared__ float lg[NT][64];
  stage_rows<float, false>(zs, z, r, tok0, nt, NT);
  __syncthreads();

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int li = lane % LPR;
  const int local = wave * (kWave / LPR) + lane / LPR;  // 0..63
  const int i = blockIdx.x * 64 + local;
  const int row_bytes = r * (WT == WT_F32 ? 4 : 2);
  const int nvec = row_bytes / 16;

  float acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = 0.0f;
  row_partial<WT, LPR, NT, 16, float>(w2_t + (size_t)i * row_bytes, nullptr, nvec, li, zs, r, acc);
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = group_sum<LPR>(acc[t]);
  if (li == 0) {
#pragma unroll
    for (int t = 0; t < NT; ++t) lg[t][local] = acc[t];
  }
  __syncthreads();

  if (wave < nt) {
    const int tok = tok0 + wave;
    const int n = blockIdx.x * 64 + lane;
    const float v = lg[wave][lane];
    const bool on = v > tau[n];
    const unsigned long long word = __ballot(on);
    if (lane == 0) mask[(size_t)tok * (f / 64) + blockIdx.x] = (uint64_t)word;
    if (logits) logits[(size_t)tok * f + n] = v;
  }
}

static int pow2_floor(int v) {
  int p = 1;
  while (p * 2 <= v) p *= 2;
  return p;
}

// Token-group size: a power of two <= kMaxNT whose staged rows fit in LDS.
static int pick_nt(int batch, int bytes_per_token) {
  int cap = kStageBytes / bytes_per_token;
  if (cap < 1) cap = 1;
  if (cap > kMaxNT) cap = kMaxNT;
  cap = pow2_floor(cap);
  int nt = 1;
  while (nt < batch && nt < cap) nt *= 2;
  return nt;
}

template <int WT, int NT>
static void pred_pass(const PredLaunch& p, int tok0, int nt, hipStream_t s) {
  using XT = typename std::conditional<WT == WT_F32, float, f16>::type;
  const int nvec1 = p.d * (int)sizeof(XT) / 16;
  const size_t sh1 = (size_t)NT * p.d * sizeof(XT);
  if (nvec1 >= 256) {
    constexpr int LPR = 64;
    const int waves = (p.r + (kWave / LPR) - 1) / (kWave / LPR);
    hipLaunchKernelGGL((k_pred1<WT, LPR, NT>), dim3((waves + 3) / 4), dim3(256), sh1, s,
                       (const uint8_t*)p.w1_t, p.x, p.z, p.d, p.r, tok0, nt);
  } else {
    constexpr int LPR = 16;
    const int waves = (p.r + (kWave / LPR) - 1) / (kWave / LPR);
    hipLaunchKernelGGL((k_pred1<WT, LPR, NT>), dim3((waves + 3) / 4), dim3(256), sh1, s,
                       (const uint8_t*)p.w1_t, p.x, p.z, p.d, p.r, tok0, nt);
  }
  const size_t sh2 = (size_t)NT * p.r * sizeof(float);
  hipLaunchKernelGGL((k_pred2<WT, NT>), dim3(p.f / 64), dim3(512), sh2, s, (const uint8_t*)p.w2_t, p.z,
                     p.tau, p.mask, p.logits, p.f, p.r, tok0, nt);
}

template <int WT>
static void pred_all(const PredLaunch& p, hipStream_t s) {
  const int xb = (WT == WT_F32) ? 4 : 2;
  int per_tok = p.d * xb;
  if (p.r * 4 > per_tok) per_tok = p.r * 4;
  const int NT = pick_nt(p.batch, per_tok);
  for (int tok0 = 0; tok0 < p.batch; tok0 += NT) {
    const int nt = (p.batch - tok0 < NT) ? (p.batch - tok0) : NT;
    switch (NT) {
      case 1: pred_pass<WT, 1>(p, tok0, nt, s); break;
      case 2: pred_pass<WT, 2>(p, tok0, nt, s); break;
      case 4: pred_pass<WT, 4>(p, tok0, nt, s); break;
      default: pred_pass<WT, 8>(p, tok0, nt, s); break;
    }
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
