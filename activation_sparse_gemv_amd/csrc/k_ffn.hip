// Neuron-gathered FFN: only the listed neurons' rows are read.
//
// A zero activation zeroes the whole row of the down projection it multiplies,
// so that row need not be loaded at all (53ai.com sparsity survey, section
// 激活稀疏); PowerInfer's GPU operators work on individual neuron rows and
// columns (same survey, PowerInfer 概述).  Storage is neuron-major: neuron i
// owns row i of W_up, W_gate and W_down^T, each a contiguous d_model run.
//
// k_ffn : one launch does the whole gathered FFN for a contiguous run of the
//         active slots per workgroup:
//   1. the run and its neuron ids come from the caller's list, from the
//      identity (dense), or from compacting the union mask in the prologue
//      (popcount + workgroup prefix sum over all mask words; no separate
//      compaction launch between the predictor and the FFN);
//   2. up (+ gate): one wavefront per neuron row, 16-byte coalesced loads,
//      activations in LDS, ReLU / ReGLU and the per-token select fused; h goes
//      to LDS;
//   3. down: every thread owns CPT consecutive output columns and adds
//      h_j * W_down^T[id_j][cols] over the run's rows in slot order.
//   The first batch of W_down^T rows is requested right behind the first up
//   loads, so both projections' rows are in flight together.  Each workgroup
//   writes one fp32 partial row per token.
// k_sum : y = b_down + the workgroups' partials in a fixed order (and
//         optionally the residual add).  No atomics anywhere, so results are
//         run-to-run deterministic.
#include "common.hpp"
#include "launch.hpp"

#ifndef SFNN_FFN_WGS
#define SFNN_FFN_WGS 256  // FFN workgroups (raised when d_ff / kMaxPer needs more)
#endif

namespace sfnn {

constexpr int kMaxPer = 512;  // slots one FFN workgroup can own

struct FfnArgs {
  const uint8_t *w_up, *w_gate, *w_down_t;
  const f16 *s_up, *s_gate, *s_down_t;
  const void *b_up, *b_gate;
  const void* x;
  const int32_t* ids;
  const int32_t* count;
  const uint64_t* union_mask;
  int32_t* ids_out;
  int32_t* count_out;
  const uint64_t* mask;  // per-token gate or null
  float* partial;        // [G][B][d]
  int d, f, B, tok0, nt, write_ids;
};

// Block-wide exclusive scan of one int per thread; returns the exclusive
// prefix and sets *total.  sh holds one int per wavefront.
template <int NTH>
__device__ __forceinline__ int block_excl_scan(int v, int* sh, int* total) {
  constexpr int NW = NTH / kWave;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  int inc = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int n = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += n;
  }
  if (lane == kWave - 1) sh[wave] = inc;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    before += (w < wave) ? sh[w] : 0;
    all += sh[w];
  }
  *total = all;
  __syncthreads();
  return before + inc - v;
}

// CPT consecutive output columns of one W_down^T row, kept in storage form
// until use (fp32: 4 B, fp16: 2 B, INT4: 1/2 B per column + the fp16 scale of
// their 128-column group).  CPT is 8, 16 or 32.
template <int WT, int CPT>
struct DownCols {
  static constexpr int NV = (WT == WT_F32) ? CPT / 4 : (WT == WT_F16 ? CPT / 8 : 1);  // 16-byte registers
  u32x4 a[NV];
  float s;

  __device__ __forceinline__ void load(const uint8_t* __restrict__ w, const f16* __restrict__ sc, int i, int col,
                                       int d) {
    if constexpr (WT == WT_F32) {
      const uint8_t* p = w + ((size_t)i * d + col) * 4;
#pragma unroll
      for (int k = 0; k < NV; ++k) a[k] = ld16_stream(p + 16 * k);
    } else if constexpr (WT == WT_F16) {
      const uint8_t* p = w + ((size_t)i * d + col) * 2;
#pragma unroll
      for (int k = 0; k < NV; ++k) a[k] = ld16_stream(p + 16 * k);
    } else {
      const uint8_t* p = w + (size_t)i * (d / 2) + col / 2;
      if constexpr (CPT == 8) {
        a[0].x = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
      } else if constexpr (CPT == 16) {
        const uint64_t q = __builtin_nontemporal_load(reinterpret_cast<const uint64_t*>(p));
        a[0].x = (uint32_t)q;
        a[0].y = (uint32_t)(q >> 32);
      } else {
        a[0] = ld16_stream(p);
      }
      s = (float)sc[(size_t)i * (d / 128) + col / 128];  // CPT <= 32 columns share one group
    }
  }

  __device__ __forceinline__ void unpack(float* w) const {
    if constexpr (WT == WT_F32) {
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        w[4 * k] = bitcast<float>(a[k].x);
        w[4 * k + 1] = bitcast<float>(a[k].y);
        w[4 * k + 2] = bitcast<float>(a[k].z);
        w[4 * k + 3] = bitcast<float>(a[k].w);
      }
    } else if constexpr (WT == WT_F16) {
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const uint32_t u[4] = {a[k].x, a[k].y, a[k].z, a[k].w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const f16x2 hh = bitcast<f16x2>(u[m]);
          w[8 * k + 2 * m] = (float)hh.x;
          w[8 * k + 2 * m + 1] = (float)hh.y;
        }
      }
    } else {
      const uint32_t u[4] = {a[0].x, a[0].y, a[0].z, a[0].w};
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        const int q = (int)(u[k >> 3] << (28 - 4 * (k & 7))) >> 28;  // sign-extended nibble
        w[k] = (float)q * s;
      }
    }
  }
};

template <int WT, int ACT, int NT, int SRC, int NTH, int CPT>
__global__ __launch_bounds__(NTH) void k_ffn(FfnArgs a) {
  using XT = typename std::conditional<WT == WT_F32, float, f16>::type;
  constexpr int NW = NTH / kWave;
  // W_down^T rows in flight per thread per buffer: 8 x 16 bytes of columns,
  // fewer where the accumulators or a 1024-thread workgroup leave few registers
  constexpr int NV = DownCols<WT, CPT>::NV;
  constexpr int kDB0 = NV >= 8 ? 1 : (NV >= 4 ? 2 : (NV == 2 ? 4 : 8));
  constexpr int kDB1 = (NT * CPT >= 64 && kDB0 > 2) ? kDB0 / 2 : kDB0;
  constexpr int kDB = kDB1 * CPT > 128 ? 128 / CPT : kDB1;
  constexpr int UB = 8;
  extern __shared__ __align__(16) unsigned char smem[];
  XT* xs = reinterpret_cast<XT*>(smem);
  __shared__ int s_ids[kMaxPer];
  __shared__ float s_h[NT][kMaxPer];
  __shared__ int s_scan[NW];
  __shared__ int s_range[2];

  const int d = a.d, f = a.f;
  const int G = gridDim.x, g = blockIdx.x;

  // ---- 1. this workgroup's run of slots and their neuron ids ---------------
  StageSplit<XT, WT == WT_I4, 2> stage;
  if constexpr (SRC == SRC_UNION) {
    // thread t owns mask words WPT*t .. WPT*t + WPT-1 (d_ff <= 65536 -> <= 1024 words)
    constexpr int WPT = 1024 / NTH;
    const int W = f / 64;
    uint64_t u[WPT];
#pragma unroll
    for (int k = 0; k < WPT; ++k) {
      const int w = WPT * threadIdx.x + k;
      u[k] = (w < W) ? a.union_mask[w] : 0ull;
    }
    stage.issue(reinterpret_cast<const XT*>(a.x), d, a.tok0, a.nt, NT);
    int pc[WPT], mine = 0;
#pragma unroll
    for (int k = 0; k < WPT; ++k) {
      pc[k] = __popcll(u[k]);
      mine += pc[k];
    }
    int total;
    const int off0 = block_excl_scan<NTH>(mine, s_scan, &total);
    const int per = (total + G - 1) / G;
    const int s0 = g * per;
    const int s1 = (s0 + per < total) ? s0 + per : total;
    int off = off0;
#pragma unroll
    for (int k = 0; k < WPT; ++k) {
      if (off < s1 && off + pc[k] > s0) {  // emit the set bits whose slots fall in [s0, s1)
        uint64_t bits = u[k];
        int slot = off;
        while (bits) {
          const int b = __builtin_ctzll(bits);
          bits &= bits - 1;
          if (slot >= s0 && slot < s1) {
            const int id = (WPT * threadIdx.x + k) * 64 + b;
            s_ids[slot - s0] = id;
            if (a.write_ids) a.ids_out[slot] = id;
          }
          ++slot;
        }
      }
      off += pc[k];
    }
    if (a.write_ids && g == 0 && threadIdx.x == 0) *a.count_out = total;
    if (threadIdx.x == 0) {
      s_range[0] = s0;
      s_range[1] = s1 > s0 ? s1 - s0 : 0;
    }
  } else {
    int n = f;
    if constexpr (SRC == SRC_IDS) {
      n = *a.count;
      n = n < 0 ? 0 : (n > f ? f : n);
    }
    const int per = (n + G - 1) / G;
    const int s0 = g * per;
    const int cnt = (s0 + per < n) ? per : (n > s0 ? n - s0 : 0);
    stage.issue(reinterpret_cast<const XT*>(a.x), d, a.tok0, a.nt, NT);
    for (int j = threadIdx.x; j < cnt; j += NTH) {
      const int id = (SRC == SRC_IDS) ? a.ids[s0 + j] : s0 + j;
      s_ids[j] = ((unsigned)id < (unsigned)f) ? id : -1;
    }
    if (threadIdx.x == 0) {
      s_range[0] = s0;
      s_range[1] = cnt;
    }
  }
  stage.commit(xs, reinterpret_cast<const XT*>(a.x), d, a.tok0, a.nt, NT);
  __syncthreads();

  const int cnt = s_range[1];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int row_bytes = (WT == WT_F32) ? d * 4 : (WT == WT_F16 ? d * 2 : d / 2);
  const int nvec = row_bytes / 16;
  const int ngroups = d / 128;
  const int words = f / 64;
  const int col0 = threadIdx.x * CPT;
  const bool colok = col0 < d;
  const int col = colok ? col0 : 0;  // keeps every address in bounds

  // ---- 2. up (+ gate) rows: one wavefront per slot -------------------------
  DownCols<WT, CPT> wd[2][kDB];
  bool first_up = true;
  for (int j = wave; j < cnt; j += NW) {  // wave-uniform loop over this workgroup's slots
    const int i = s_ids[j];
    const bool ok = i >= 0;
    const int ic = ok ? i : 0;
    float au[NT], ag[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) au[t] = ag[t] = 0.0f;
    const uint8_t* ru = a.w_up + (size_t)ic * row_bytes;
    const f16* su = a.s_up ? a.s_up + (size_t)ic * ngroups : nullptr;
    const uint8_t* rg = (ACT == ACT_REGLU) ? a.w_gate + (size_t)ic * row_bytes : nullptr;
    const f16* sg = (ACT == ACT_REGLU && a.s_gate) ? a.s_gate + (size_t)ic * ngroups : nullptr;
    for (int v0 = lane; v0 < nvec; v0 += UB * kWave) {
      RowLoads<WT, kWave, UB> Lu, Lg;
      Lu.issue(ru, su, nvec, v0);
      if constexpr (ACT == ACT_REGLU) Lg.issue(rg, sg, nvec, v0);
      if (first_up) {
        // the first W_down^T batch goes out right behind this wave's first up loads
#pragma unroll
        for (int u = 0; u < kDB; ++u) {
          const int jj = u < cnt ? u : 0;
          const int iu = s_ids[jj];
          wd[0][u].load(a.w_down_t, a.s_down_t, iu >= 0 ? iu : 0, col, d);
        }
        first_up = false;
      }
      __builtin_amdgcn_sched_barrier(0);  // every load above is issued before any math
      Lu.template consume<NT>(nvec, v0, xs, d, au);
      if constexpr (ACT == ACT_REGLU) Lg.template consume<NT>(nvec, v0, xs, d, ag);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      au[t] = group_sum<kWave>(au[t]);
      if (ACT == ACT_REGLU) ag[t] = group_sum<kWave>(ag[t]);
    }
    // lane t finishes token t
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (lane == t) {
        float hv = 0.0f;
        if (ok && t < a.nt) {
          const float up = au[t] + (a.b_up ? load_as_float<XT>(a.b_up, i) : 0.0f);
          if (ACT == ACT_RELU) {
            hv = up > 0.0f ? up : 0.0f;
          } else {
            const float gt = ag[t] + (a.b_gate ? load_as_float<XT>(a.b_gate, i) : 0.0f);
            hv = (gt > 0.0f ? gt : 0.0f) * up;
          }
          if (a.mask) {
            const uint64_t wv = a.mask[(size_t)(a.tok0 + t) * words + (i >> 6)];
            if (!((wv >> (i & 63)) & 1ull)) hv = 0.0f;  // select: gated-off neurons add nothing
          }
        }
        s_h[t][j] = hv;
      }
    }
  }
  if (first_up) {  // waves without an up row still bring in the first W_down^T batch
#pragma unroll
    for (int u = 0; u < kDB; ++u) {
      const int jj = u < cnt ? u : 0;
      const int iu = cnt > 0 ? s_ids[jj] : 0;
      wd[0][u].load(a.w_down_t, a.s_down_t, iu >= 0 ? iu : 0, col, d);
    }
  }
  __syncthreads();

  // ---- 3. down: acc[t][k] += h[t][j] * W_down^T[id_j][col + k], slots in order
  float acc[NT][CPT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int k = 0; k < CPT; ++k) acc[t][k] = 0.0f;

  for (int j0 = 0; j0 < cnt; j0 += 2 * kDB) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int jb = j0 + half * kDB;  // batch held in buffer `half`
      if (jb < cnt) {
        // request the batch after this one into the other buffer
        const int jn = jb + kDB;
        if (jn < cnt) {
#pragma unroll
          for (int u = 0; u < kDB; ++u) {
            const int jj = (jn + u < cnt) ? jn + u : jn;
            const int iu = s_ids[jj];
            wd[half ^ 1][u].load(a.w_down_t, a.s_down_t, iu >= 0 ? iu : 0, col, d);
          }
        }
#pragma unroll
        for (int u = 0; u < kDB; ++u) {
          const int jj = jb + u;
          const int jc = jj < cnt ? jj : jb;
          const bool ok = jj < cnt && s_ids[jc] >= 0 && colok;
          float wf[CPT];
          wd[half][u].unpack(wf);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const float hv = ok ? s_h[t][jc] : 0.0f;
#pragma unroll
            for (int k = 0; k < CPT; ++k) acc[t][k] = __builtin_fmaf(hv, ok ? wf[k] : 0.0f, acc[t][k]);
          }
        }
      }
    }
  }

  if (colok) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t < a.nt) {
        float* dst = a.partial + ((size_t)g * a.B + a.tok0 + t) * d + col0;
#pragma unroll
        for (int k = 0; k < CPT; k += 4) {
          const f32x4 v = f32x4{acc[t][k], acc[t][k + 1], acc[t][k + 2], acc[t][k + 3]};
          // streamed past L2: the sum kernel reads it once, and the end of
          // this kernel need not write back megabytes of dirty lines
          __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(dst + k));
        }
      }
    }
  }
}

// y[e] = b_down[c] + sum over workgroups g = 0..G-1 of partial[g][e], e = t*d + c:
// 16 elements per workgroup; thread (q, c) adds the g's of group q in order,
// then the 16 group sums are added in order.  With r_in: r_out = r_in + y.
template <typename XT>
__global__ __launch_bounds__(256) void k_sum(const float* __restrict__ partial, int G, int B, int d,
                                             const void* __restrict__ b_down, float* __restrict__ y,
                                             const float* __restrict__ r_in, float* __restrict__ r_out) {
  constexpr int EPW = 16, NQ = 16, BAT = 16;
  __shared__ float part[NQ][EPW];
  const int c16 = threadIdx.x % EPW, q = threadIdx.x / EPW;
  const int n = B * d;
  const int e = blockIdx.x * EPW + c16;
  const int ec = e < n ? e : 0;
  const int per = (G + NQ - 1) / NQ;
  const int g0 = q * per;
  const int g1 = (g0 + per < G) ? g0 + per : G;
  float s = 0.0f;
  for (int b0 = g0; b0 < g1; b0 += BAT) {
    float p[BAT];
#pragma unroll
    for (int j = 0; j < BAT; ++j) {
      const int gg = (b0 + j < g1) ? b0 + j : b0;
      p[j] = partial[(size_t)gg * n + ec];
    }
#pragma unroll
    for (int j = 0; j < BAT; ++j)
      if (b0 + j < g1) s += p[j];
  }
  part[q][c16] = s;
  __syncthreads();
  if (q == 0 && e < n) {
    const int c = e % d;
    float v = b_down ? load_as_float<XT>(b_down, c) : 0.0f;
    float tot = 0.0f;
#pragma unroll
    for (int k = 0; k < NQ; ++k) tot += part[k][c16];
    v += tot;
    if (y) y[e] = v;
    if (r_in) r_out[e] = r_in[e] + v;
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

struct FfnShape {
  int cpt, nth, nt;
};

// Threads own CPT columns each for the down projection (at most 512
// threads); the token group is bounded by the staged activations (LDS) and by
// 64 accumulators per thread.
static FfnShape ffn_shape(int wt, int d, int batch) {
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

template <int WT, int ACT, int NT, int NTH, int CPT>
static void ffn_pass(const FfnLaunch& p, int tok0, int nt, bool first, hipStream_t s) {
  using XT = typename std::conditional<WT == WT_F32, float, f16>::type;
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
  a.d = p.d;
  a.f = p.f;
  a.B = p.batch;
  a.tok0 = tok0;
  a.nt = nt;
  a.write_ids = (p.src == SRC_UNION && first) ? 1 : 0;
  const size_t sh = (size_t)NT * p.d * sizeof(XT);
  const int G = p.groups;
  if (p.src == SRC_UNION)
    hipLaunchKernelGGL((k_ffn<WT, ACT, NT, SRC_UNION, NTH, CPT>), dim3(G), dim3(NTH), sh, s, a);
  else if (p.src == SRC_IDS)
    hipLaunchKernelGGL((k_ffn<WT, ACT, NT, SRC_IDS, NTH, CPT>), dim3(G), dim3(NTH), sh, s, a);
  else
    hipLaunchKernelGGL((k_ffn<WT, ACT, NT, SRC_DENSE, NTH, CPT>), dim3(G), dim3(NTH), sh, s, a);
}

template <int WT, int ACT, int NT, int NTH>
static void ffn_pass_cpt(const FfnLaunch& p, int cpt, int tok0, int nt, bool first, hipStream_t s) {
  if (cpt == 8)
    ffn_pass<WT, ACT, NT, NTH, 8>(p, tok0, nt, first, s);
  else if (cpt == 16)
    ffn_pass<WT, ACT, (NT > 4 ? 4 : NT), NTH, 16>(p, tok0, nt, first, s);
  else
    ffn_pass<WT, ACT, (NT > 2 ? 2 : NT), NTH, 32>(p, tok0, nt, first, s);
}

template <int WT, int ACT, int NT>
static void ffn_pass_nth(const FfnLaunch& p, const FfnShape& sh, int tok0, int nt, bool first, hipStream_t s) {
  if (sh.nth == 256)
    ffn_pass<WT, ACT, NT, 256, 8>(p, tok0, nt, first, s);  // 256 threads only when d <= 2048, CPT 8
  else
    ffn_pass_cpt<WT, ACT, NT, 512>(p, sh.cpt, tok0, nt, first, s);
}

template <int WT, int ACT>
static void ffn_all(const FfnLaunch& p, hipStream_t s) {
  using XT = typename std::conditional<WT == WT_F32, float, f16>::type;
  const FfnShape sh = ffn_shape(WT, p.d, p.batch);
  for (int tok0 = 0; tok0 < p.batch; tok0 += sh.nt) {
    const int nt = (p.batch - tok0 < sh.nt) ? (p.batch - tok0) : sh.nt;
    const bool first = tok0 == 0;
    switch (sh.nt) {
      case 1: ffn_pass_nth<WT, ACT, 1>(p, sh, tok0, nt, first, s); break;
      case 2: ffn_pass_nth<WT, ACT, 2>(p, sh, tok0, nt, first, s); break;
      case 4: ffn_pass_nth<WT, ACT, 4>(p, sh, tok0, nt, first, s); break;
      default: ffn_pass_nth<WT, ACT, 8>(p, sh, tok0, nt, first, s); break;
    }
  }
  if (p.y || p.r_out) {
    const int n = p.batch * p.d;
    hipLaunchKernelGGL((k_sum<XT>), dim3((n + 15) / 16), dim3(256), 0, s, p.partial, p.groups, p.batch, p.d,
                       p.b_down, p.y, p.r_in, p.r_out);
  }
}

hipError_t launch_ffn(const FfnLaunch& p, hipStream_t s) {
  if (p.act == ACT_RELU) {
    if (p.wt == WT_F32) ffn_all<WT_F32, ACT_RELU>(p, s);
    else if (p.wt == WT_F16) ffn_all<WT_F16, ACT_RELU>(p, s);
    else ffn_all<WT_I4, ACT_RELU>(p, s);
  } else {
    if (p.wt == WT_F32) ffn_all<WT_F32, ACT_REGLU>(p, s);
    else if (p.wt == WT_F16) ffn_all<WT_F16, ACT_REGLU>(p, s);
    else ffn_all<WT_I4, ACT_REGLU>(p, s);
  }
  return hipGetLastError();
}

}  // namespace sfnn
