// Neuron-gathered FFN: only the listed neurons' rows are read.
//
// A zero activation zeroes the whole row of the down projection it multiplies,
// so that row need not be loaded at all (53ai.com sparsity survey, section
// 激活稀疏); PowerInfer's GPU operators work on individual neuron rows and
// columns (same survey, PowerInfer 概述).  Storage is neuron-major: neuron i
// owns row i of W_up, W_gate and W_down^T, each a contiguous d_model run.
//
// k_up   : gather-GEMV.  One wavefront per neuron row, 16-byte coalesced loads,
//          activations staged in LDS, ReLU / ReGLU and the per-token gate fused;
//          writes h[tok][slot] (fp32).
// k_down : column-scatter down projection.  Workgroup (tile, row block) sums
//          h * W_down^T[ids] over its block of slots for 256 output columns and
//          writes one fp32 partial per row block.
// k_reduce: y = b_down + the row-block partials added in row-block order.  No
//          atomics anywhere, so results are run-to-run deterministic.
#include "common.hpp"
#include "launch.hpp"

namespace sfnn {

constexpr int kTile = 256;   // output columns per down-projection workgroup

template <int WT, int ACT, int NT>
__global__ __launch_bounds__(256) void k_up(
    const uint8_t* __restrict__ w_up, const uint8_t* __restrict__ w_gate, const f16* __restrict__ s_up,
    const f16* __restrict__ s_gate, const void* __restrict__ b_up, const void* __restrict__ b_gate,
    const void* __restrict__ x, const int32_t* __restrict__ ids, const int32_t* __restrict__ count,
    const uint64_t* __restrict__ mask, float* __restrict__ h, int d, int f, int tok0, int nt) {
  using XT = typename std::conditional<WT == WT_F32, float, f16>::type;
  extern __shared__ __align__(16) unsigned char smem[];
  XT* xs = reinterpret_cast<XT*>(smem);
  int n = f;
  if (ids) {
    n = *count;
    n = n < 0 ? 0 : (n > f ? f : n);
  }
  // workgroups past the last listed neuron have nothing to do
  if ((int)(blockIdx.x * (blockDim.x / kWave)) >= n) return;
  stage_rows<XT, WT == WT_I4>(xs, reinterpret_cast<const XT*>(x), d, tok0, nt, NT);
  __syncthreads();
  const int lane = threadIdx.x & (kWave - 1);
  const int gw = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int GW = gridDim.x * (blockDim.x / kWave);
  const int row_bytes = (WT == WT_F32) ? d * 4 : (WT == WT_F16 ? d * 2 : d / 2);
  const int nvec = row_bytes / 16;
  const int ngroups = d / 128;
  const int words = f / 64;

  for (int slot = gw; slot < n; slot += GW) {  // wave-uniform loop
    const int i = ids ? ids[slot] : slot;
    const bool ok = (unsigned)i < (unsigned)f;
    float au[NT], ag[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) au[t] = ag[t] = 0.0f;
    if (ok) {
      row_partial<WT, kWave, NT, 8, XT>(w_up + (size_t)i * row_bytes, s_up ? s_up + (size_t)i * ngroups : nullptr,
                                      nvec, lane, xs, d, au);
      if (ACT == ACT_REGLU)
        row_partial<WT, kWave, NT, 8, XT>(w_gate + (size_t)i * row_bytes,
                                        s_gate ? s_gate + (size_t)i * ngroups : nullptr, nvec, lane, xs, d, ag);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      au[t] = group_sum<kWave>(au[t]);
      if (ACT == ACT_REGLU) ag[t] = group_sum<kWave>(ag[t]);
    }
    // lane t finishes token t
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (lane == t && t < nt) {
        float hv = 0.0f;
        if (ok) {
          const float up = au[t] + (b_up ? load_as_float<XT>(b_up, i) : 0.0f);
          if (ACT == ACT_RELU) {
            hv = up > 0.0f ? up : 0.0f;
          } else {
            const float g = ag[t] + (b_gate ? load_as_float<XT>(b_gate, i) : 0.0f);
            hv = (g > 0.0f ? g : 0.0f) * up;
          }
          if (mask) {
            const uint64_t wv = mask[(size_t)(tok0 + t) * words + (i >> 6)];
            if (!((wv >> (i & 63)) & 1ull)) hv = 0.0f;
          }
        }
        h[(size_t)(tok0 + t) * f + slot] = hv;
      }
    }
  }
}

// Eight consecutive output columns of one W_down^T row as fp32.
template <int WT>
__device__ __forceinline__ void load8(const uint8_t* __restrict__ w_down_t, const f16* __restrict__ s_down_t,
                                      int i, int col, int d, float* w) {
  if constexpr (WT == WT_F32) {
    const uint8_t* p = w_down_t + ((size_t)i * d + col) * 4;
    const u32x4 a = ld16_stream(p), b = ld16_stream(p + 16);
    w[0] = bitcast<float>(a.x); w[1] = bitcast<float>(a.y); w[2] = bitcast<float>(a.z); w[3] = bitcast<float>(a.w);
    w[4] = bitcast<float>(b.x); w[5] = bitcast<float>(b.y); w[6] = bitcast<float>(b.z); w[7] = bitcast<float>(b.w);
  } else if constexpr (WT == WT_F16) {
    const u32x4 a = ld16_stream(w_down_t + ((size_t)i * d + col) * 2);
    const uint32_t u[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const f16x2 hh = bitcast<f16x2>(u[k]);
      w[2 * k] = (float)hh.x;
      w[2 * k + 1] = (float)hh.y;
    }
  } else {
    const uint32_t u = __builtin_nontemporal_load(
        reinterpret_cast<const uint32_t*>(w_down_t + (size_t)i * (d / 2) + col / 2));
    const float s = (float)s_down_t[(size_t)i * (d / 128) + col / 128];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int q = (int)(u << (28 - 4 * k)) >> 28;  // sign-extended nibble k
      w[k] = (float)q * s;
    }
  }
}

constexpr int kChunk = 256;  // slots staged in LDS per step of the down projection
constexpr int kUnroll = 4;   // independent row loads in flight per lane

template <int WT, int NT>
__global__ __launch_bounds__(256) void k_down(const uint8_t* __restrict__ w_down_t,
                                              const f16* __restrict__ s_down_t, const float* __restrict__ h,
                                              const int32_t* __restrict__ ids, const int32_t* __restrict__ count,
                                              float* __restrict__ partial, int d, int f, int tok0, int nt) {
  __shared__ float red[4][NT][kTile];
  __shared__ int s_ids[kChunk];
  __shared__ float s_h[NT][kChunk];
  const int tile = blockIdx.x, rb = blockIdx.y, R = gridDim.y;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int rg = wave * 2 + (lane >> 5);          // row group 0..7
  const int cl = (lane & 31) * 8;                 // column offset inside the tile
  const int col0 = tile * kTile + cl;
  const bool colok = col0 < d;
  const int col = colok ? col0 : 0;               // keeps every address in bounds

  int n = f;
  if (ids) {
    n = *count;
    n = n < 0 ? 0 : (n > f ? f : n);
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
      const int i = ids ? ids[c0 + j] : c0 + j;
      s_ids[j] = ((unsigned)i < (unsigned)f) ? i : -1;
#pragma unroll
      for (int t = 0; t < NT; ++t) s_h[t][j] = (t < nt) ? h[(size_t)(tok0 + t) * f + c0 + j] : 0.0f;
    }
    __syncthreads();
    const int ilast = s_ids[cn - 1];
    for (int j = rg; j < cn; j += 8 * kUnroll) {
      float w[kUnroll][8];
      bool ok[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int jj = j + 8 * u;
        const int iu = jj < cn ? s_ids[jj] : ilast;  // tail slots re-read a row this block loads anyway
        ok[u] = (jj < cn) && (iu >= 0) && colok;
        load8<WT>(w_down_t, s_down_t, iu >= 0 ? iu : 0, col, d, w[u]);
      }
      __builtin_amdgcn_sched_barrier(0);  // all row loads of the batch issue before any FMA
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int jj = (j + 8 * u < cn) ? j + 8 * u : cn - 1;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const float hv = s_h[t][jj];
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const float wk = ok[u] ? w[u][k] : 0.0f;  // select: skipped rows add exactly nothing
            acc[t][k] = __builtin_fmaf(ok[u] ? hv : 0.0f, wk, acc[t][k]);
          }
        }
      }
    }
    __syncthreads();
  }
  // lanes l and l+32 hold the same columns for neighbouring row groups
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[t][k] += __shfl_xor(acc[t][k], 32, kWave);
  if (lane < 32) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int k = 0; k < 8; ++k) red[wave][t][cl + k] = acc[t][k];
  }
  __syncthreads();
  const int c = tile * kTile + threadIdx.x;
  if (c < d) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t < nt) {
        const float v = ((red[0][t][threadIdx.x] + red[1][t][threadIdx.x]) + red[2][t][threadIdx.x]) +
                        red[3][t][threadIdx.x];
        partial[((size_t)rb * kMaxNT + t) * d + c] = v;
      }
    }
  }
}

// y[tok][c] = b_down[c] + sum over row blocks q = 0..R-1 (in order) of partial[q][t][c].
template <typename XT>
__global__ __launch_bounds__(64) void k_reduce(const float* __restrict__ partial, const void* __restrict__ b_down,
                                               float* __restrict__ y, int d, int R, int tok0, int nt) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;  // (t, c) pairs
  if (e >= nt * d) return;
  const int t = e / d, c = e - t * d;
  float v = b_down ? load_as_float<XT>(b_down, c) : 0.0f;
  for (int q0 = 0; q0 < R; q0 += 16) {
    float p[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int q = (q0 + j < R) ? q0 + j : q0;
      p[j] = partial[((size_t)q * kMaxNT + t) * d + c];
    }
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (q0 + j < R) v += p[j];
  }
  y[(size_t)(tok0 + t) * d + c] = v;
}

int ffn_row_blocks(int d, int f) {
  const int tiles = (d + kTile - 1) / kTile;
  int R = (512 + tiles - 1) / tiles;
  if (R < 4) R = 4;
  if (R > 64) R = 64;
  if (R > f / 8) R = f / 8 > 0 ? f / 8 : 1;
  return R;
}

template <int WT, int ACT, int NT>
static void ffn_pass(const FfnLaunch& p, int tok0, int nt, hipStream_t s) {
  using XT = typename std::conditional<WT == WT_F32, float, f16>::type;
  const int ntiles = (p.d + kTile - 1) / kTile;
  const size_t sh = (size_t)NT * p.d * sizeof(XT);
  int blocks = (p.f + 3) / 4;  // one wave per neuron slot at most
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL((k_up<WT, ACT, NT>), dim3(blocks), dim3(256), sh, s, (const uint8_t*)p.w_up,
                     (const uint8_t*)p.w_gate, (const f16*)p.s_up, (const f16*)p.s_gate, p.b_up, p.b_gate, p.x,
                     p.ids, p.count, p.mask, p.h, p.d, p.f, tok0, nt);
  hipLaunchKernelGGL((k_down<WT, NT>), dim3(ntiles, p.row_blocks), dim3(256), 0, s, (const uint8_t*)p.w_down_t,
                     (const f16*)p.s_down_t, p.h, p.ids, p.count, p.partial, p.d, p.f, tok0, nt);
  hipLaunchKernelGGL((k_reduce<XT>), dim3((nt * p.d + 63) / 64), dim3(64), 0, s, p.partial, p.b_down, p.y, p.d,
                     p.row_blocks, tok0, nt);
}

template <int WT, int ACT>
static void ffn_all(const FfnLaunch& p, hipStream_t s) {
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
    switch (NT) {
      case 1: ffn_pass<WT, ACT, 1>(p, tok0, nt, s); break;
      case 2: ffn_pass<WT, ACT, 2>(p, tok0, nt, s); break;
      case 4: ffn_pass<WT, ACT, 4>(p, tok0, nt, s); break;
      default: ffn_pass<WT, ACT, 8>(p, tok0, nt, s); break;
    }
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
