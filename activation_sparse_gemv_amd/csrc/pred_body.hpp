// Workgroup bodies of the low-rank activation predictor:
// z = W1^T x, logit = W2^T z, mask = logit > tau.
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
//   pred1_body: one wavefront per row of W1^T, x staged in LDS.  In a
//     residual stack the prologue builds x = r / rms(r) from the residual row.
//   pred2_body: a workgroup owns 64 neurons (one mask word per token); each
//     wavefront takes 8 rows of W2^T with all 64 lanes on every row and z held
//     in registers, so z is read once per lane instead of once per row; the 8
//     row sums come out of one multi-row butterfly.  The threshold is fused,
//     64 decisions are packed per __ballot and the batch's words are ORed into
//     the union mask.
// The bodies take a virtual workgroup index so that a launch can run them
// beside other work (the look-ahead stack fuses them with the FFN).
#pragma once
#include "common.hpp"
#include "launch.hpp"

namespace sfnn {

constexpr int kChainMaxV = 16;  // float4 vectors of the residual rows kept per thread (at most)

// Residual-chain prologue, issue half: this thread's float4 vectors of the
// nt residual rows.  Slot (t, k) holds vector threadIdx.x + k * blockDim.x of
// token t's row, k < CV / NT.  Requires d / 4 <= (CV / NT) * blockDim.x
// (checked on the host).
// UNCOND = false: slots past the row load nothing and hold zeros; use it where
// many slots are spare (redundant loads of one shared address serialise in
// the cache).  The loads sit in branches, so a later wait for anything
// issued before them also waits for them.
// UNCOND = true (slot count sized to the shape): every slot loads, spare ones
// re-read the row's last vector or token tok0's row, and chain_finish masks
// them; with no branch, waits for earlier loads stop short of these.
template <int NT, int CV, bool UNCOND = false>
__device__ __forceinline__ void chain_issue(const float* __restrict__ r_in, f32x4 (&v)[CV], int d, int tok0,
                                            int nt) {
  constexpr int KPT = CV / NT;
  const int nv = d / 4;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
      const int c4 = threadIdx.x + k * blockDim.x;
      if constexpr (UNCOND) {
        const int tc = t < nt ? t : 0;
        const int cc = c4 < nv ? c4 : nv - 1;
        v[t * KPT + k] = *reinterpret_cast<const f32x4*>(r_in + (size_t)(tok0 + tc) * d + 4 * cc);
      } else {
        v[t * KPT + k] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (t < nt && c4 < nv)
          v[t * KPT + k] = *reinterpret_cast<const f32x4*>(r_in + (size_t)(tok0 + t) * d + 4 * c4);
      }
    }
  }
}

// Finish half: x = r / sqrt(mean(r^2) + eps) rounded to XT into xs (and, if
// x_out is given and `writer`, into x_out).  Every workgroup of a launch sums
// in the same fixed order (thread, lane scan, wavefront), so all get the same
// x.  red holds NT x (waves) floats.  PERM8 stores xs in the INT4 pairing
// order inside every 8-element vector (x0 x4 x1 x5 x2 x6 x3 x7); x_out is
// always in natural order.  Rows of tokens >= nt stage zeros.
template <typename XT, int NT, bool PERM8, int CV>
__device__ __forceinline__ void chain_finish(const f32x4 (&v)[CV], XT* xs, float (*red)[16], void* x_out,
                                             bool writer, float eps, int d, int tok0, int nt) {
  constexpr int KPT = CV / NT;
  const int nv = d / 4;
  const int nw = blockDim.x / kWave;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
      const bool ok = t < nt && (int)threadIdx.x + k * (int)blockDim.x < nv;  // spare slots add nothing
      const f32x4 q = ok ? v[t * KPT + k] : f32x4{0.f, 0.f, 0.f, 0.f};
      ss = __builtin_fmaf(q.x, q.x, ss);
      ss = __builtin_fmaf(q.y, q.y, ss);
      ss = __builtin_fmaf(q.z, q.z, ss);
      ss = __builtin_fmaf(q.w, q.w, ss);
    }
    ss = wave_sum(ss);
    if (lane == 0) red[t][wave] = ss;
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float tot = 0.0f;
    for (int w = 0; w < nw; ++w) tot += red[t][w];
    const float sc = 1.0f / __builtin_sqrtf(tot / (float)d + eps);
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
      const int c4 = threadIdx.x + k * blockDim.x;
      if (c4 < nv) {
        const f32x4 o = t < nt ? v[t * KPT + k] * sc : f32x4{0.f, 0.f, 0.f, 0.f};  // tokens >= nt stage zeros
        const XT o0 = (XT)o.x, o1 = (XT)o.y, o2 = (XT)o.z, o3 = (XT)o.w;
        if constexpr (PERM8) {
          // elements 4h..4h+3 of an 8-vector go to positions h, h+2, h+4, h+6
          XT* dst = xs + (size_t)t * d + 8 * (c4 >> 1) + (c4 & 1);
          dst[0] = o0;
          dst[2] = o1;
          dst[4] = o2;
          dst[6] = o3;
        } else {
          XT* dst = xs + (size_t)t * d + 4 * c4;
          dst[0] = o0;
          dst[1] = o1;
          dst[2] = o2;
          dst[3] = o3;
        }
        if (writer && x_out && t < nt) {
          XT* xo = reinterpret_cast<XT*>(x_out) + (size_t)(tok0 + t) * d + 4 * c4;
          xo[0] = o0;
          xo[1] = o1;
          xo[2] = o2;
          xo[3] = o3;
        }
      }
    }
  }
}

struct Pred1Args {
  const uint8_t* w1_t;  // [r][d]
  const void* x;        // [B][d] plain input (when norm.r_in is null)
  NormIn norm;
  float* z;             // [B][r]
  int d, r, tok0, nt;
};

// Stage 1 for virtual workgroup vb of vg: z[tok][j] = sum_k w1_t[j][k] x[tok][k].
template <int WT, int LPR, int NT, bool CHAIN>
__device__ __forceinline__ void pred1_body(const Pred1Args& a, int vb, int vg) {
  using XT = typename std::conditional<WT == WT_F32, float, f16>::type;
  constexpr int UB = 8;
  constexpr int RPW = kWave / LPR;  // rows per wave per step
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ float red[NT][16];
  XT* xs = reinterpret_cast<XT*>(smem);
  const int d = a.d, r = a.r;

  const int lane = threadIdx.x & (kWave - 1);
  const int li = lane % LPR;
  const int gw = vb * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int GW = vg * (blockDim.x / kWave);
  const int row_bytes = d * (int)sizeof(XT);
  const int nvec = row_bytes / 16;

  // activations first, then this lane group's first batch of its first row
  f32x4 rv[kChainMaxV];
  StageSplit<XT, false, 2> stage;
  if constexpr (CHAIN)
    chain_issue<NT, kChainMaxV>(a.norm.r_in, rv, d, a.tok0, a.nt);
  else
    stage.issue(reinterpret_cast<const XT*>(a.x), d, a.tok0, a.nt, NT);
  // keep the activation loads ahead of the weight loads: vector loads return
  // in order, so the staging below then waits for the activations only
  __builtin_amdgcn_sched_barrier(0);
  // Unconditional issue (a lane without a first row re-reads row 0): a
  // branch here would make the wait in the prologue below cover these loads.
  RowLoads<WT, LPR, UB> L;
  const int j0 = gw * RPW + lane / LPR;
  const bool pre = j0 < r && li < nvec;
  L.issue(a.w1_t + (size_t)(pre ? j0 : 0) * row_bytes, nullptr, nvec, pre ? li : 0);
  __builtin_amdgcn_sched_barrier(0);  // and the prologue's math after all of them
  if constexpr (CHAIN)
    chain_finish<XT, NT, false, kChainMaxV>(rv, xs, red, a.norm.x_out, vb == 0, a.norm.eps, d, a.tok0, a.nt);
  else
    stage.commit(xs, reinterpret_cast<const XT*>(a.x), d, a.tok0, a.nt, NT);
  __syncthreads();

  for (int base = gw * RPW; base < r; base += GW * RPW) {
    const int j = base + lane / LPR;
    float acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = 0.0f;
    if (j < r)
      row_dot<WT, LPR, UB, NT, XT>(L, pre && base == gw * RPW, a.w1_t + (size_t)j * row_bytes, nullptr, nvec, li,
                                   xs, d, acc);
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = group_sum<LPR>(acc[t]);
    if (li == 0 && j < r) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
        if (t < a.nt) a.z[(size_t)(a.tok0 + t) * r + j] = acc[t];
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

struct Pred2Args {
  const uint8_t* w2_t;  // [f][r]
  const float* z;       // [B][r]
  const float* tau;     // [f]
  uint64_t* mask;       // [B][f/64]
  uint64_t* union_mask; // [f/64]
  float* logits;        // [B][f] or null
  int f, r, tok0, nt, first_pass;
  int hot;              // mask words [0, hot) form the dense hot prefix
};

// Stage 2 for mask word vb: 8 waves (512 threads) of 8 rows; VPL 16-byte
// vectors per lane per row; RB rows in flight per wave.  In two phases so
// that a fused launch can issue other loads between them: issue() sends z,
// tau and the first RB rows' weights, finish() adds them up (loading the
// rest, when RB < 8), thresholds and writes the mask words.  Dense hot-prefix
// words are the caller's (pred2_hot_word).
template <int WT, int NT, int VPL, int RB>
struct Pred2Tile {
  static constexpr int E = vec_elems<WT>();  // 4 (fp32) or 8 (fp16) weights per vector
  f32x4 zf[NT][VPL][E / 4];
  u32x4 w[RB][VPL];
  float tv;

  __device__ __forceinline__ void load_rows(const Pred2Args& a, int vb, int rb0) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int row_bytes = a.r * (WT == WT_F32 ? 4 : 2);
    const int nvec = row_bytes / 16;
#pragma unroll
    for (int k = 0; k < RB; ++k) {
      const int i = vb * 64 + wave * 8 + rb0 + k;
#pragma unroll
      for (int u = 0; u < VPL; ++u) {
        const int v = lane + kWave * u;
        w[k][u] = ld16_stream(a.w2_t + (size_t)i * row_bytes + 16 * (size_t)(v < nvec ? v : 0));
      }
    }
  }

  // z elements of this lane's vectors (lane + 64u), straight to registers.
  // Out-of-range vectors and tokens read an in-bounds z element and are
  // cancelled later (zero weights / unused token), so nothing here waits for
  // the loads and the weight loads go out right behind them.
  __device__ __forceinline__ void issue(const Pred2Args& a, int vb) {
    const int lane = threadIdx.x & (kWave - 1);
    const int r = a.r;
    const int nvec = r * (WT == WT_F32 ? 4 : 2) / 16;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int u = 0; u < VPL; ++u) {
        const int v = lane + kWave * u;
        const bool ok = v < nvec && t < a.nt;
        const float* src = a.z + (size_t)(a.tok0 + (t < a.nt ? t : 0)) * r + (size_t)(ok ? v : 0) * E;
#pragma unroll
        for (int q = 0; q < E / 4; ++q) zf[t][u][q] = *reinterpret_cast<const f32x4*>(src + 4 * q);
      }
    tv = a.tau[vb * 64 + lane];
    load_rows(a, vb, 0);
  }

  // write == false: the same loads, math and barriers, no output (a
  // workgroup of a fused launch with no mask word of its own)
  __device__ __forceinline__ void finish(const Pred2Args& a, int vb, bool write = true) {
    __shared__ float lg[NT][64];
    __shared__ unsigned long long wsh[NT];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int f = a.f;
    const int nvec = a.r * (WT == WT_F32 ? 4 : 2) / 16;
#pragma unroll
    for (int rb0 = 0; rb0 < 8; rb0 += RB) {
      if (rb0 > 0) load_rows(a, vb, rb0);
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

    if (write && wave < a.nt) {
      const int tok = a.tok0 + wave;
      const float v = lg[wave][lane];
      const bool on = v > tv;
      const unsigned long long word = __ballot(on);
      if (lane == 0) {
        a.mask[(size_t)tok * (f / 64) + vb] = (uint64_t)word;
        wsh[wave] = word;
      }
      if (a.logits) a.logits[(size_t)tok * f + vb * 64 + lane] = v;
    }
    __syncthreads();
    if (write && threadIdx.x == 0) {
      uint64_t u = a.first_pass ? 0ull : a.union_mask[vb];
      for (int t = 0; t < a.nt; ++t) u |= wsh[t];
      a.union_mask[vb] = u;
    }
  }
};

template <int WT, int NT, int VPL, int RB>
__device__ __forceinline__ void pred2_body(const Pred2Args& a, int vb) {
  if (vb < a.hot) {  // uniform over the workgroup: no barrier below is reached
    pred2_hot_word(a.mask, a.union_mask, a.logits, a.f, a.tok0, a.nt, vb);
    return;
  }
  Pred2Tile<WT, NT, VPL, RB> P;
  P.issue(a, vb);
  P.finish(a, vb);
}

// Token-group and shape choices and argument builders shared by the launchers.
int pred_group(int wt, int d, int r, int batch, bool chain);
int pred2_vpl(int wt, int r);
int pred2_group(int wt, int r, int batch);
Pred1Args pred1_args(const PredLaunch& p, int tok0, int nt);
Pred2Args pred2_args(const PredLaunch& p, int tok0, int nt);

}  // namespace sfnn
