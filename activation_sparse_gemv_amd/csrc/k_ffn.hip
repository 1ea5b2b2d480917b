// Neuron-gathered FFN: only the listed neurons' rows are read.
//
// A zero activation zeroes the whole row of the down projection it multiplies,
// so that row need not be loaded at all (53ai.com sparsity survey, section
// 激活稀疏); PowerInfer's GPU operators work on individual neuron rows and
// columns (same survey, PowerInfer 概述).  Storage is neuron-major: neuron i
// owns row i of W_up, W_gate and W_down^T, each a contiguous d_model run.
//
// k_up   : gather-GEMV.  Workgroup g takes a contiguous run of the active
//          slots; its ids come from the caller's list, from the identity
//          (dense), or from compacting the union mask in the prologue (every
//          workgroup prefix-sums the mask words in LDS, so no separate
//          compaction launch sits between the predictor and the FFN).  One
//          wavefront per neuron row, 16-byte coalesced loads, activations in
//          LDS, ReLU / ReGLU and the per-token gate fused; writes h[tok][slot].
// k_down : column-scatter down projection.  Workgroup (tile, row block) sums
//          h * W_down^T[ids] over its run of slots for one column tile and
//          writes one fp32 partial per row block.
// k_reduce: y = b_down + the row-block partials added in row-block order (and
//          optionally the residual add).  No atomics anywhere, so results are
//          run-to-run deterministic.
#include "common.hpp"
#include "launch.hpp"

#ifndef SFNN_DOWN_LPR
#define SFNN_DOWN_LPR 16  // lanes per W_down^T row fragment (8 columns per lane)
#endif
#ifndef SFNN_DOWN_UB
#define SFNN_DOWN_UB 8    // row fragments in flight per lane
#endif
#ifndef SFNN_DOWN_WGS
#define SFNN_DOWN_WGS 512  // target workgroups of the down projection
#endif
#ifndef SFNN_UP_WGS
#define SFNN_UP_WGS 512    // workgroups of the up projection (fewer if d_ff is small)
#endif

namespace sfnn {

constexpr int kUpMaxPer = 128;  // slots one up-projection workgroup can own
constexpr int kChunk = 256;     // slots staged in LDS per step of the down projection

struct UpArgs {
  const uint8_t *w_up, *w_gate;
  const f16 *s_up, *s_gate;
  const void *b_up, *b_gate;
  const void* x;
  const int32_t* ids;
  const int32_t* count;
  const uint64_t* union_mask;
  int32_t* ids_out;
  int32_t* count_out;
  const uint64_t* mask;  // per-token gate or null
  float* h;
  int d, f, tok0, nt, write_ids;
};

// Block-wide exclusive scan of one int per thread (256 threads); returns the
// exclusive prefix and sets *total.
__device__ __forceinline__ int block_excl_scan256(int v, int* sh, int* total) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  int inc = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int n = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += n;
  }
  if (lane == kWave - 1) sh[wave] = inc;
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) before += (w < wave) ? sh[w] : 0;
  *total = (sh[0] + sh[1]) + (sh[2] + sh[3]);
  __syncthreads();
  return before + inc - v;
}

template <int WT, int ACT, int NT, int SRC>
__global__ __launch_bounds__(256) void k_up(UpArgs a) {
  using XT = typename std::conditional<WT == WT_F32, float, f16>::type;
  constexpr int UB = 8;
  extern __shared__ __align__(16) unsigned char smem[];
  XT* xs = reinterpret_cast<XT*>(smem);
  __shared__ int s_ids[kUpMaxPer];
  __shared__ int s_scan[4];
  __shared__ int s_range[2];

  const int d = a.d, f = a.f;
  const int G = gridDim.x, g = blockIdx.x;

  // ---- which slots this workgroup owns, and their neuron ids ----------------
  if constexpr (SRC == SRC_UNION) {
    // thread t owns mask words 4t .. 4t+3 (d_ff <= 65536 -> <= 1024 words)
    const int W = f / 64;
    uint64_t u[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int w = 4 * threadIdx.x + k;
      u[k] = (w < W) ? a.union_mask[w] : 0ull;
    }
    stage_rows<XT, WT == WT_I4>(xs, reinterpret_cast<const XT*>(a.x), d, a.tok0, a.nt, NT);
    int pc[4], mine = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      pc[k] = __popcll(u[k]);
      mine += pc[k];
    }
    int total;
    const int off0 = block_excl_scan256(mine, s_scan, &total);
    const int per = (total + G - 1) / G;
    const int s0 = g * per;
    const int s1 = (s0 + per < total) ? s0 + per : total;
    int off = off0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      // emit the set bits of word 4t+k whose slots fall in [s0, s1)
      if (off < s1 && off + pc[k] > s0) {
        uint64_t bits = u[k];
        int slot = off;
        while (bits) {
          const int b = __builtin_ctzll(bits);
          bits &= bits - 1;
          if (slot >= s0 && slot < s1) {
            const int id = (4 * threadIdx.x + k) * 64 + b;
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
    int id = -1;
    if (threadIdx.x < cnt) id = (SRC == SRC_IDS) ? a.ids[s0 + threadIdx.x] : s0 + threadIdx.x;
    stage_rows<XT, WT == WT_I4>(xs, reinterpret_cast<const XT*>(a.x), d, a.tok0, a.nt, NT);
    if (threadIdx.x < cnt) s_ids[threadIdx.x] = id;
    if (threadIdx.x == 0) {
      s_range[0] = s0;
      s_range[1] = cnt;
    }
  }
  __syncthreads();

  const int s0 = s_range[0], cnt = s_range[1];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int row_bytes = (WT == WT_F32) ? d * 4 : (WT == WT_F16 ? d * 2 : d / 2);
  const int nvec = row_bytes / 16;
  const int ngroups = d / 128;
  const int words = f / 64;

  for (int j = wave; j < cnt; j += 4) {  // wave-uniform loop over this workgroup's slots
    const int i = s_ids[j];
    const bool ok = (unsigned)i < (unsigned)f;
    const int ic = ok ? i : 0;
    float au[NT], ag[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) au[t] = ag[t] = 0.0f;
    if (ok) {
      RowLoads<WT, kWave, UB> Lu, Lg;
      const uint8_t* ru = a.w_up + (size_t)ic * row_bytes;
      const f16* su = a.s_up ? a.s_up + (size_t)ic * ngroups : nullptr;
      const uint8_t* rg = (ACT == ACT_REGLU) ? a.w_gate + (size_t)ic * row_bytes : nullptr;
      const f16* sg = (ACT == ACT_REGLU && a.s_gate) ? a.s_gate + (size_t)ic * ngroups : nullptr;
      for (int v0 = lane; v0 < nvec; v0 += UB * kWave) {
        Lu.issue(ru, su, nvec, v0);
        if constexpr (ACT == ACT_REGLU) Lg.issue(rg, sg, nvec, v0);
        __builtin_amdgcn_sched_barrier(0);  // both rows' loads ahead of the math
        Lu.template consume<NT>(nvec, v0, xs, d, au);
        if constexpr (ACT == ACT_REGLU) Lg.template consume<NT>(nvec, v0, xs, d, ag);
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      au[t] = group_sum<kWave>(au[t]);
      if (ACT == ACT_REGLU) ag[t] = group_sum<kWave>(ag[t]);
    }
    // lane t finishes token t
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (lane == t && t < a.nt) {
        float hv = 0.0f;
        if (ok) {
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
        a.h[(size_t)(a.tok0 + t) * f + s0 + j] = hv;
      }
    }
  }
}

// Eight consecutive output columns of one W_down^T row, kept in their storage
// form until use (fp32: 32 bytes, fp16: 16 bytes, INT4: 4 bytes + the scale
// of their 128-column group) so that many rows fit in flight per lane.
template <int WT>
struct Cols8 {
  u32x4 a, b;
  float s;
  __device__ __forceinline__ void load(const uint8_t* __restrict__ w_down_t, const f16* __restrict__ s_down_t, int i,
                                       int col, int d) {
    if constexpr (WT == WT_F32) {
      const uint8_t* p = w_down_t + ((size_t)i * d + col) * 4;
      a = ld16_stream(p);
      b = ld16_stream(p + 16);
    } else if constexpr (WT == WT_F16) {
      a = ld16_stream(w_down_t + ((size_t)i * d + col) * 2);
    } else {
      a.x = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(w_down_t + (size_t)i * (d / 2) + col / 2));
      s = (float)s_down_t[(size_t)i * (d / 128) + col / 128];
    }
  }
  __device__ __forceinline__ void unpack(float* w) const {
    if constexpr (WT == WT_F32) {
      w[0] = bitcast<float>(a.x); w[1] = bitcast<float>(a.y); w[2] = bitcast<float>(a.z); w[3] = bitcast<float>(a.w);
      w[4] = bitcast<float>(b.x); w[5] = bitcast<float>(b.y); w[6] = bitcast<float>(b.z); w[7] = bitcast<float>(b.w);
    } else if constexpr (WT == WT_F16) {
      const uint32_t u[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const f16x2 hh = bitcast<f16x2>(u[k]);
        w[2 * k] = (float)hh.x;
        w[2 * k + 1] = (float)hh.y;
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int q = (int)(a.x << (28 - 4 * k)) >> 28;  // sign-extended nibble k
        w[k] = (float)q * s;
      }
    }
  }
};

struct DownArgs {
  const uint8_t* w_down_t;
  const f16* s_down_t;
  const float* h;
  const int32_t* ids;    // null: dense (slot = neuron)
  const int32_t* count;  // null: dense
  float* partial;        // [R][B][d]
  int d, f, B, tok0, nt;
};

// Workgroup (tile, rb): columns [tile*TW, tile*TW + TW), slots of row block rb.
// Lane group rg (LPR lanes) of wave wv takes rows rg + RPW*wv + 4*RPW*k; each
// lane owns 8 columns.
template <int WT, int NT, int LPR, int UB>
__global__ __launch_bounds__(256) void k_down(DownArgs a) {
  constexpr int RPW = kWave / LPR;
  constexpr int TW = LPR * 8;
  constexpr int RSTEP = 4 * RPW;
  __shared__ int s_ids[kChunk];
  __shared__ float s_h[NT][kChunk];
  __shared__ float red[4][NT][TW];
  const int tile = blockIdx.x, rb = blockIdx.y, R = gridDim.y;
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  const int li = lane % LPR, rg = lane / LPR;
  const int row0 = wv * RPW + rg;
  const int col0 = tile * TW + li * 8;
  const bool colok = col0 < a.d;
  const int col = colok ? col0 : 0;  // keeps every address in bounds

  int n = a.f;
  if (a.count) {
    n = *a.count;
    n = n < 0 ? 0 : (n > a.f ? a.f : n);
  }
  const int per = (n + R - 1) / R;
  const int s0 = rb * per;
  const int s1 = (s0 + per < n) ? s0 + per : n;

  float acc[NT][8];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[t][k] = 0.0f;

  for (int c0 = s0; c0 < s1; c0 += kChunk) {
    const int cn = (s1 - c0 < kChunk) ? s1 - c0 : kChunk;
    for (int j = threadIdx.x; j < cn; j += blockDim.x) {
      const int i = a.ids ? a.ids[c0 + j] : c0 + j;
      s_ids[j] = ((unsigned)i < (unsigned)a.f) ? i : -1;
#pragma unroll
      for (int t = 0; t < NT; ++t) s_h[t][j] = (t < a.nt) ? a.h[(size_t)(a.tok0 + t) * a.f + c0 + j] : 0.0f;
    }
    __syncthreads();
    for (int j = row0; j < cn; j += UB * RSTEP) {
      Cols8<WT> w[UB];
      bool ok[UB];
      const int ifirst = s_ids[j];
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const int jj = j + u * RSTEP;
        const int iu = jj < cn ? s_ids[jj] : ifirst;  // tail slots re-read a row this lane loads anyway
        ok[u] = (jj < cn) && (iu >= 0) && colok;
        w[u].load(a.w_down_t, a.s_down_t, iu >= 0 ? iu : 0, col, a.d);
      }
      __builtin_amdgcn_sched_barrier(0);  // all row loads of the batch issue before any FMA
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const int jj = (j + u * RSTEP < cn) ? j + u * RSTEP : j;
        float wf[8];
        w[u].unpack(wf);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const float hv = ok[u] ? s_h[t][jj] : 0.0f;
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const float wk = ok[u] ? wf[k] : 0.0f;  // select: skipped rows add exactly nothing
            acc[t][k] = __builtin_fmaf(hv, wk, acc[t][k]);
          }
        }
      }
    }
    __syncthreads();
  }
  // lanes with the same li in the wave's RPW row groups hold the same columns
#pragma unroll
  for (int m = LPR; m < kWave; m <<= 1)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[t][k] += __shfl_xor(acc[t][k], m, kWave);
  if (rg == 0) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int k = 0; k < 8; ++k) red[wv][t][li * 8 + k] = acc[t][k];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < NT * TW; e += blockDim.x) {
    const int t = e / TW, cc = e - t * TW;
    const int c = tile * TW + cc;
    if (t < a.nt && c < a.d) {
      const float v = ((red[0][t][cc] + red[1][t][cc]) + red[2][t][cc]) + red[3][t][cc];
      a.partial[((size_t)rb * a.B + a.tok0 + t) * a.d + c] = v;
    }
  }
}

// y[t][c] = b_down[c] + sum over row blocks q = 0..R-1 (in order) of partial[q][t][c];
// with r_in: r_out = r_in + y.
template <typename XT>
__global__ __launch_bounds__(64) void k_reduce(const float* __restrict__ partial, const void* __restrict__ b_down,
                                                float* __restrict__ y, const float* __restrict__ r_in,
                                                float* __restrict__ r_out, int d, int R, int B) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;  // (t, c) pairs
  if (e >= B * d) return;
  const int c = e % d;
  float v = b_down ? load_as_float<XT>(b_down, c) : 0.0f;
  for (int q0 = 0; q0 < R; q0 += 16) {
    float p[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int q = (q0 + j < R) ? q0 + j : q0;
      p[j] = partial[(size_t)q * B * d + e];
    }
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (q0 + j < R) v += p[j];
  }
  if (y) y[e] = v;
  if (r_in) r_out[e] = r_in[e] + v;
}

// Row blocks of the down projection: enough workgroups to fill the chip.
int ffn_row_blocks(int wt, int d, int f) {
  (void)wt;
  constexpr int TW = SFNN_DOWN_LPR * 8;
  const int tiles = (d + TW - 1) / TW;
  int R = (SFNN_DOWN_WGS + tiles - 1) / tiles;
  if (R < 1) R = 1;
  if (R > 64) R = 64;
  if (R > f / 8) R = f / 8 > 0 ? f / 8 : 1;
  return R;
}

static int up_grid(int f) {
  int G = SFNN_UP_WGS;
  const int need = (f + kUpMaxPer - 1) / kUpMaxPer;  // every slot must fit some workgroup's LDS list
  if (G < need) G = need;
  if (G > f / 4) G = f / 4 > need ? f / 4 : need;
  return G;
}

template <int WT, int ACT, int NT>
static void ffn_pass(const FfnLaunch& p, int tok0, int nt, bool first, hipStream_t s) {
  using XT = typename std::conditional<WT == WT_F32, float, f16>::type;
  constexpr int LPR = SFNN_DOWN_LPR;
  constexpr int TW = LPR * 8;
  const int ntiles = (p.d + TW - 1) / TW;
  const size_t sh = (size_t)NT * p.d * sizeof(XT);
  UpArgs ua;
  ua.w_up = (const uint8_t*)p.w_up;
  ua.w_gate = (const uint8_t*)p.w_gate;
  ua.s_up = (const f16*)p.s_up;
  ua.s_gate = (const f16*)p.s_gate;
  ua.b_up = p.b_up;
  ua.b_gate = p.b_gate;
  ua.x = p.x;
  ua.ids = p.ids;
  ua.count = p.count;
  ua.union_mask = p.union_mask;
  ua.ids_out = p.ids_out;
  ua.count_out = p.count_out;
  ua.mask = p.mask;
  ua.h = p.h;
  ua.d = p.d;
  ua.f = p.f;
  ua.tok0 = tok0;
  ua.nt = nt;
  ua.write_ids = (p.src == SRC_UNION && first) ? 1 : 0;
  const int G = up_grid(p.f);
  if (p.src == SRC_UNION)
    hipLaunchKernelGGL((k_up<WT, ACT, NT, SRC_UNION>), dim3(G), dim3(256), sh, s, ua);
  else if (p.src == SRC_IDS)
    hipLaunchKernelGGL((k_up<WT, ACT, NT, SRC_IDS>), dim3(G), dim3(256), sh, s, ua);
  else
    hipLaunchKernelGGL((k_up<WT, ACT, NT, SRC_DENSE>), dim3(G), dim3(256), sh, s, ua);

  DownArgs da;
  da.w_down_t = (const uint8_t*)p.w_down_t;
  da.s_down_t = (const f16*)p.s_down_t;
  da.h = p.h;
  da.ids = p.src == SRC_DENSE ? nullptr : (p.src == SRC_UNION ? p.ids_out : p.ids);
  da.count = p.src == SRC_DENSE ? nullptr : (p.src == SRC_UNION ? p.count_out : p.count);
  da.partial = p.partial;
  da.d = p.d;
  da.f = p.f;
  da.B = p.batch;
  da.tok0 = tok0;
  da.nt = nt;
  constexpr int DUB = NT <= 2 ? SFNN_DOWN_UB : (NT <= 4 ? (SFNN_DOWN_UB > 4 ? SFNN_DOWN_UB / 2 : SFNN_DOWN_UB) : (SFNN_DOWN_UB > 4 ? SFNN_DOWN_UB / 4 : 2));
  hipLaunchKernelGGL((k_down<WT, NT, LPR, DUB>), dim3(ntiles, p.row_blocks), dim3(256), 0, s, da);
}

template <int WT, int ACT>
static void ffn_all(const FfnLaunch& p, hipStream_t s) {
  using XT = typename std::conditional<WT == WT_F32, float, f16>::type;
  const int xb = (WT == WT_F32) ? 4 : 2;
  int cap = kStageBytes / (p.d * xb);
  if (cap < 1) cap = 1;
  if (cap > kMaxNT) cap = kMaxNT;
  int c2 = 1;
  while (c2 * 2 <= cap) c2 *= 2;
  int NT = 1;
  while (NT < p.batch && NT < c2) NT *= 2;
  for (int tok0 = 0; tok0 < p.batch; tok0 += NT) {
    const int nt = (p.batch - tok0 < NT) ? (p.batch - tok0) : NT;
    const bool first = tok0 == 0;
    switch (NT) {
      case 1: ffn_pass<WT, ACT, 1>(p, tok0, nt, first, s); break;
      case 2: ffn_pass<WT, ACT, 2>(p, tok0, nt, first, s); break;
      case 4: ffn_pass<WT, ACT, 4>(p, tok0, nt, first, s); break;
      default: ffn_pass<WT, ACT, 8>(p, tok0, nt, first, s); break;
    }
  }
  if (p.y) {
    const int n = p.batch * p.d;
    hipLaunchKernelGGL((k_reduce<XT>), dim3((n + 63) / 64), dim3(64), 0, s, p.partial, p.b_down, p.y,
                       (const float*)nullptr, (float*)nullptr, p.d, p.row_blocks, p.batch);
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

hipError_t launch_reduce(const float* partial, int R, int batch, int d, const void* b_down, int xtype, float* y,
                         const float* r_in, float* r_out, hipStream_t s) {
  const int n = batch * d;
  if (xtype == WT_F32)
    hipLaunchKernelGGL((k_reduce<float>), dim3((n + 63) / 64), dim3(64), 0, s, partial, b_down, y, r_in, r_out,
                       d, R, batch);
  else
    hipLaunchKernelGGL((k_reduce<f16>), dim3((n + 63) / 64), dim3(64), 0, s, partial, b_down, y, r_in, r_out,
                       d, R, batch);
  return hipGetLastError();
}

}  // namespace sfnn
