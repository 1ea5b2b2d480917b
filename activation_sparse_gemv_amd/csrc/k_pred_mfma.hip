// The low-rank predictor of larger batches on the matrix cores (fp16
// predictor weights).
//
// The predictor is a dense chain over every neuron ([53ai] 自适应稀疏预测器:
// a small network in front of each FFN that guesses the active neurons):
// z = W1^T x, logits = W2^T z, active iff logit > tau.  The VALU kernels hold
// at most a few tokens per pass and re-read W1 and W2 once per token group;
// here one pass covers up to 32 tokens with v_mfma_f32_16x16x32_f16, fp32
// accumulation.
//
//  k_pred1_mfma  workgroup = 16 rows of W1^T x one of up to 8 d_model
//                slices (enough for one batch of pairs per wavefront); its
//                16 wavefronts split the
//                slice into 64-column pairs (pair w, w + 16, ...), each
//                holding a 16x16 fp32 block per 16 tokens; the blocks are
//                added in wavefront order in LDS and written as the slice's
//                partial z, which k_z_reduce adds in slice order into z
//                [B][r] fp32.
//  k_pred2_mfma  workgroup = 64 neurons (one mask word, four 16-row tiles) x
//                every token of the pass; its 8 wavefronts split the rank
//                into 32-wide steps (step w, w + 8, ...).  z enters the
//                matrix cores as two fp16 planes (hi = fp16(z), lo =
//                fp16(z - hi)), so the logits keep 22 bits of z, far inside
//                the predictor's fp32 error band.  Blocks added in wavefront
//                order, then threshold, one ballot per token and mask word,
//                union OR.
//
// Every sum is taken in a fixed order, so the results are run-to-run
// bitwise deterministic, and on integer inputs below 2^22 they are exact.
#include "common.hpp"
#include "launch.hpp"

namespace sfnn {

// Stage 1 has only r / 16 workgroups, so each runs 16 wavefronts; both stages
// keep kPredBatch iterations of loads in flight per wavefront.
constexpr int kPred1Waves = 16;
constexpr int kPredBatch = 4;

struct Pred1MfmaArgs {
  const f16* w1_t;  // [r][d]
  const f16* x;     // [B][d]
  float* z;         // [B][r] (one slice), or the slices' partial z [KS][B][r]
  int d, r, B, tok0, nt, KS;
};

struct Pred2MfmaArgs {
  const f16* w2_t;        // [f][r]
  const float* z;         // [B][r]
  const float* tau;       // [f]
  uint64_t* mask;         // [B][f/64]
  uint64_t* union_mask;   // [f/64]
  float* logits;          // [B][f] or null
  int f, r, tok0, nt, first_pass;
  int hot;                // mask words [0, hot) form the dense hot prefix
};

template <int NB>
struct P1Frag {
  u32x4 w[2];      // [K block of the pair]
  u32x4 x[NB][2];  // [token tile][K block]
};

template <int NB>
__global__ __launch_bounds__(1024) void k_pred1_mfma(Pred1MfmaArgs a) {
  __shared__ f32x4 red[kPred1Waves][NB][kWave];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int rr = lane & 15, g = lane >> 4;
  const int d = a.d;
  const int tile = blockIdx.x / a.KS, ks = blockIdx.x % a.KS;  // row tile, d_model slice
  const int row = tile * 16 + rr;
  const f16* wr = a.w1_t + (size_t)(row < a.r ? row : a.r - 1) * d + 8 * g;  // rows past r: dropped below
  const f16* xr[NB];
  bool xok[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int tk = nb * 16 + rr;
    xok[nb] = tk < a.nt;
    xr[nb] = a.x + (size_t)(a.tok0 + (xok[nb] ? tk : 0)) * d + 8 * g;
  }
  f32x4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto issue = [&](P1Frag<NB>& F, int pair) {
    const int k = pair * 64;
#pragma unroll
    for (int s = 0; s < 2; ++s) F.w[s] = ld16_stream(wr + k + 32 * s);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int s = 0; s < 2; ++s) F.x[nb][s] = ld16(xr[nb] + k + 32 * s);
  };
  auto mul = [&](const P1Frag<NB>& F) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[nb] = mfma_16x16x32(F.w[s], xok[nb] ? F.x[nb][s] : zero, acc[nb]);
  };

  // this slice's pairs p0 + wave, + W, ... in batches of kPredBatch: every
  // batch's loads go out before any of its products (a pair past the last
  // re-reads the last)
  constexpr int W = kPred1Waves;
  const int npair = d >> 6;
  const int p0 = ks * npair / a.KS, p1 = (ks + 1) * npair / a.KS;
  const int iters = p0 + wave < p1 ? (p1 - p0 - wave + W - 1) / W : 0;
  for (int b0 = 0; b0 < iters; b0 += kPredBatch) {
    P1Frag<NB> F[kPredBatch];
#pragma unroll
    for (int j = 0; j < kPredBatch; ++j) issue(F[j], p0 + wave + W * (b0 + j < iters ? b0 + j : iters - 1));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < kPredBatch; ++j)
      if (b0 + j < iters) mul(F[j]);
  }

#pragma unroll
  for (int nb = 0; nb < NB; ++nb) red[wave][nb][lane] = acc[nb];
  __syncthreads();
  constexpr int E = NB * kWave * 4;  // floats per wavefront's blocks
  const int e = threadIdx.x;
  if (e < E) {
    const float* rf = reinterpret_cast<const float*>(&red[0][0][0]);
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < kPred1Waves; ++w) s += rf[w * E + e];
    const int q = e & 3, ln = (e >> 2) & (kWave - 1), nb = e >> 8;
    const int orow = tile * 16 + 4 * (ln >> 4) + q;
    const int tk = nb * 16 + (ln & 15);
    if (orow < a.r && tk < a.nt) a.z[((size_t)ks * a.B + a.tok0 + tk) * a.r + orow] = s;
  }
}

// z = the slices' partial z added in slice order, for elements [e0, e1) of
// [B][r].
__global__ __launch_bounds__(256) void k_z_reduce(const float* __restrict__ zpart, int KS, int n, int e0, int e1,
                                                  float* __restrict__ z) {
  const int e = e0 + blockIdx.x * 256 + threadIdx.x;
  if (e >= e1) return;
  float s = zpart[e];
  for (int k = 1; k < KS; ++k) s += zpart[(size_t)k * n + e];
  z[e] = s;
}

template <int NB>
__global__ __launch_bounds__(512) void k_pred2_mfma(Pred2MfmaArgs a) {
  __shared__ f32x4 red[8][2][NB][kWave];  // two row tiles at a time
  __shared__ unsigned char bits[32][64];  // [token][neuron of the word]
  __shared__ unsigned long long wsh[32];
  if ((int)blockIdx.x < a.hot) {  // uniform over the workgroup
    pred2_hot_word(a.mask, a.union_mask, a.logits, a.f, a.tok0, a.nt, blockIdx.x);
    return;
  }
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int rr = lane & 15, g = lane >> 4;
  const int r = a.r;
  const int n0 = blockIdx.x * 64;
  const f16* wr[4];  // row starts
#pragma unroll
  for (int t = 0; t < 4; ++t) wr[t] = a.w2_t + (size_t)(n0 + t * 16 + rr) * r;
  const float* zr[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int tk = nb * 16 + rr;
    zr[nb] = a.z + (size_t)(a.tok0 + (tk < a.nt ? tk : 0)) * r;
  }
  bool zok[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) zok[nb] = nb * 16 + rr < a.nt;
  // thresholds of the logits this thread sums after the reduction (tile pair
  // tp, e-slot k), fetched now so that no load waits at the end
  float tv[2][NB];
#pragma unroll
  for (int tp = 0; tp < 2; ++tp)
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int e = threadIdx.x + 512 * k;
      const int q = e & 3, ln = (e >> 2) & (kWave - 1), i = e / (256 * NB);
      tv[tp][k] = a.tau[n0 + (2 * tp + i) * 16 + 4 * (ln >> 4) + q];
    }
  f32x4 acc[4][NB];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[t][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // K block of step ks for this lane: 32 ks + 8 g; the rank is a multiple of
  // 8, so a block is either whole or past the row (then the row's first block
  // is read and zeroed: every load is unconditional and in bounds)
  struct Raw {
    u32x4 w[4];
    f32x4 z[NB][2];
  };
  auto issue = [&](Raw& R, int ks) {
    const int kb = 32 * ks + 8 * g;
    const int kc = kb < r ? kb : 0;
#pragma unroll
    for (int t = 0; t < 4; ++t) R.w[t] = ld16_stream(wr[t] + kc);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      R.z[nb][0] = *reinterpret_cast<const f32x4*>(zr[nb] + kc);
      R.z[nb][1] = *reinterpret_cast<const f32x4*>(zr[nb] + kc + 4);
    }
  };
  auto mul = [&](const Raw& R, int ks) {
    const bool ok = 32 * ks + 8 * g < r;
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      u32x4 hi, lo;
      split_hi_lo(R.z[nb][0], R.z[nb][1], hi, lo);
      if (!ok || !zok[nb]) {
        hi = zero;
        lo = zero;
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const u32x4 wv = ok ? R.w[t] : zero;
        acc[t][nb] = mfma_16x16x32(wv, hi, acc[t][nb]);
        acc[t][nb] = mfma_16x16x32(wv, lo, acc[t][nb]);
      }
    }
  };

  // steps wave, wave + 8, ... in batches of kPredBatch: every batch's loads go
  // out before any of its products (a step past the last re-reads the last)
  const int nks = (r + 31) >> 5;
  const int iters = wave < nks ? (nks - wave + 7) >> 3 : 0;
  for (int b0 = 0; b0 < iters; b0 += kPredBatch) {
    Raw R[kPredBatch];
#pragma unroll
    for (int j = 0; j < kPredBatch; ++j) issue(R[j], wave + 8 * (b0 + j < iters ? b0 + j : iters - 1));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < kPredBatch; ++j)
      if (b0 + j < iters) mul(R[j], wave + 8 * (b0 + j));
  }

  // add the 8 wavefronts' blocks in order, two row tiles at a time; thread
  // e-slots e = threadIdx.x + 512 k (k < NB) cover 2 tiles x 16 NB tokens
  constexpr int E = 2 * NB * kWave * 4;
  const float* rf = reinterpret_cast<const float*>(&red[0][0][0][0]);
#pragma unroll
  for (int tp = 0; tp < 2; ++tp) {
    if (tp) __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) red[wave][i][nb][lane] = acc[2 * tp + i][nb];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int e = threadIdx.x + 512 * k;
      float s = 0.0f;
#pragma unroll
      for (int w = 0; w < 8; ++w) s += rf[w * E + e];
      const int q = e & 3, ln = (e >> 2) & (kWave - 1), nb = (e >> 8) % NB, i = e / (256 * NB);
      const int nrow = (2 * tp + i) * 16 + 4 * (ln >> 4) + q;  // neuron within the word
      const int tk = nb * 16 + (ln & 15);
      if (tk < a.nt) {
        const int n = n0 + nrow;
        bits[tk][nrow] = s > tv[tp][k] ? 1 : 0;
        if (a.logits) a.logits[(size_t)(a.tok0 + tk) * a.f + n] = s;
      }
    }
  }
  __syncthreads();
  const int words = a.f >> 6;
  for (int tk = wave; tk < a.nt; tk += 8) {
    const unsigned long long word = __ballot(bits[tk][lane] != 0);
    if (lane == 0) {
      a.mask[(size_t)(a.tok0 + tk) * words + blockIdx.x] = (uint64_t)word;
      wsh[tk] = word;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t u = a.first_pass ? 0ull : a.union_mask[blockIdx.x];
    for (int t = 0; t < a.nt; ++t) u |= wsh[t];
    a.union_mask[blockIdx.x] = u;
  }
}

// ---- host side ---------------------------------------------------------------

bool pred_uses_mfma(const PredLaunch& p) { return p.wt == WT_F16 && p.batch >= kPredMfmaMinBatch; }

// The residual chain's layer input first (x = r / rms(r), written to x_out),
// then stage 1 on it.
hipError_t launch_pred1_mfma(const PredLaunch& p, hipStream_t s) {
  const void* x = p.x;
  if (p.norm.r_in) {
    const hipError_t e = launch_residual_rmsnorm(p.norm.r_in, nullptr, nullptr, p.batch, p.d, p.norm.eps,
                                                 p.norm.x_out, WT_F16, s);
    if (e != hipSuccess) return e;
    x = p.norm.x_out;
  }
  // d_model slices: just enough that every wavefront has one batch of pairs
  // (a slice's extra reduce launch costs more than a second batch saves when
  // d_model is small: one slice at 4096, three at 12288)
  const int tiles = (p.r + 15) / 16, npair = p.d / 64;
  int KS = (npair + kPred1Waves * kPredBatch - 1) / (kPred1Waves * kPredBatch);
  if (KS > kPred1MaxSplits) KS = kPred1MaxSplits;
  if (KS < 1 || !p.zpart) KS = 1;
  Pred1MfmaArgs a;
  a.w1_t = (const f16*)p.w1_t;
  a.x = (const f16*)x;
  a.z = KS > 1 ? p.zpart : p.z;
  a.d = p.d;
  a.r = p.r;
  a.B = p.batch;
  a.KS = KS;
  const dim3 grid(tiles * KS);
  for (int tok0 = 0; tok0 < p.batch; tok0 += 32) {
    a.tok0 = tok0;
    a.nt = p.batch - tok0 < 32 ? p.batch - tok0 : 32;
    if (a.nt > 16)
      hipLaunchKernelGGL(k_pred1_mfma<2>, grid, dim3(64 * kPred1Waves), 0, s, a);
    else
      hipLaunchKernelGGL(k_pred1_mfma<1>, grid, dim3(64 * kPred1Waves), 0, s, a);
  }
  if (KS > 1) {
    const int n = p.batch * p.r;
    hipLaunchKernelGGL(k_z_reduce, dim3((n + 255) / 256), dim3(256), 0, s, p.zpart, KS, n, 0, n, p.z);
  }
  return hipGetLastError();
}

hipError_t launch_pred2_mfma(const PredLaunch& p, hipStream_t s) {
  Pred2MfmaArgs a;
  a.w2_t = (const f16*)p.w2_t;
  a.z = p.z;
  a.tau = p.tau;
  a.mask = p.mask;
  a.union_mask = p.union_mask;
  a.logits = p.logits;
  a.f = p.f;
  a.r = p.r;
  a.hot = p.hot;
  const dim3 grid(p.f / 64);
  for (int tok0 = 0; tok0 < p.batch; tok0 += 32) {
    a.tok0 = tok0;
    a.nt = p.batch - tok0 < 32 ? p.batch - tok0 : 32;
    a.first_pass = tok0 == 0 ? 1 : 0;
    if (a.nt > 16)
      hipLaunchKernelGGL(k_pred2_mfma<2>, grid, dim3(512), 0, s, a);
    else
      hipLaunchKernelGGL(k_pred2_mfma<1>, grid, dim3(512), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace sfnn
