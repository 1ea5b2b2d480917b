// Workgroup bodies of the neuron-gathered FFN: only the listed neurons' rows
// are read.
//
// A zero activation zeroes the whole row of the down projection it multiplies,
// so that row need not be loaded at all (53ai.com sparsity survey, section
// 激活稀疏); PowerInfer's GPU operators work on individual neuron rows and
// columns (same survey, PowerInfer 概述).  Storage is neuron-major: neuron i
// owns row i of W_up, W_gate and W_down^T, each a contiguous d_model run.
//
// ffn_body: one workgroup does the whole gathered FFN for a contiguous run of
//         the active slots:
//   1. the run and its neuron ids come from the caller's list, from the
//      identity (dense), or from compacting the union mask in the prologue
//      (popcounts + a lane prefix sum over all mask words in every
//      wavefront; no separate compaction launch between the predictor and
//      the FFN);
//   2. up (+ gate): one wavefront per neuron row, 16-byte coalesced loads,
//      activations in LDS, ReLU / ReGLU and the per-token select fused; h goes
//      to LDS;
//   3. down: every thread owns CPT consecutive output columns and adds
//      h_j * W_down^T[id_j][cols] over the run's rows in slot order.
//   The first batch of W_down^T rows is requested right behind the first up
//   loads, so both projections' rows are in flight together.  Each workgroup
//   writes one fp32 partial row per token.
// sum_body: y = b_down + the workgroups' partials in a fixed order (and
//         optionally the residual add).  No atomics anywhere, so results are
//         run-to-run deterministic.
// The bodies take a virtual workgroup index so that a launch can run them
// beside other work (the look-ahead stack fuses them with the predictor).
#pragma once
#include "common.hpp"
#include "launch.hpp"
#include "pred_body.hpp"

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
  const float* r_in;     // residual rows (chain prologue: x = r / rms(r)) or null
  void* x_out;           // chain prologue: x written here by workgroup 0 (or null)
  float eps;
  const uint8_t* w1_t;   // P1: the next layer's predictor W1^T [r][d] (stage 1 on the same x)
  float* z;              // P1: its output [B][r]
  int r;                 // P1: rank (0: no predictor rows)
  int d, f, B, tok0, nt, write_ids;
};

// CPT consecutive output columns of one W_down^T row, kept in storage form
// until use (fp32: 4 B, fp16: 2 B, INT4: 1/2 B per column + the fp16 scale of
// their 128-column group).  CPT is 8, 16 or 32.
template <int WT, int CPT>
struct DownCols {
  static constexpr int NV = (WT == WT_F32) ? CPT / 4 : (WT == WT_F16 ? CPT / 8 : 1);  // 16-byte loads
  static constexpr int NQ = (WT == WT_I4) ? CPT / 8 : 1;                            // INT4: dwords held
  u32x4 a[WT == WT_I4 ? 1 : NV];
  uint32_t q[NQ];
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
        q[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
      } else if constexpr (CPT == 16) {
        const uint64_t v = __builtin_nontemporal_load(reinterpret_cast<const uint64_t*>(p));
        q[0] = (uint32_t)v;
        q[1] = (uint32_t)(v >> 32);
      } else {
        const u32x4 v = ld16_stream(p);
        q[0] = v.x;
        q[1] = v.y;
        q[2] = v.z;
        q[3] = v.w;
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
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        const int n = (int)(q[k >> 3] << (28 - 4 * (k & 7))) >> 28;  // sign-extended nibble
        w[k] = (float)n * s;
      }
    }
  }
};

// One FFN workgroup (virtual index vb of vg).  CHAIN: the layer input is
// x = r_in / rms(r_in), built in the prologue instead of staged from a.x.
// P1: the workgroup also computes its share of predictor stage 1 of the next
// layer on the same x (look-ahead): rows [vb*pr, vb*pr + pr) of W1^T, taken by
// the wavefronts from the last one down.
// Every wavefront derives the workgroup's slot list by itself (mask words,
// popcounts, one lane scan, then the 64 bits of each word that holds slots
// of the run emitted by the 64 lanes at once into the wavefront's own LDS
// list), so no workgroup barrier stands between the mask and the first
// weight loads: the barriers that stage x come after those loads are issued.
template <int WT, int ACT, int NT, int SRC, int NTH, int CPT, bool CHAIN, bool P1, int UW>
__device__ __forceinline__ void ffn_body(const FfnArgs& a, int vb, int vg) {
  using XT = typename std::conditional<WT == WT_F32, float, f16>::type;
  static_assert(!P1 || SRC == SRC_UNION, "predictor rows ride along with the union-mask FFN only");
  constexpr int NW = NTH / kWave;
  // W_down^T rows in flight per thread per buffer: 8 x 16 bytes of columns,
  // fewer where the accumulators leave few registers
  constexpr int NV = DownCols<WT, CPT>::NV;
  constexpr int kDB0 = NV >= 8 ? 1 : (NV >= 4 ? 2 : (NV == 2 ? 4 : 8));
  constexpr int kDB1 = (NT * CPT >= 64 && kDB0 > 2) ? kDB0 / 4 : ((NT * CPT >= 32 && kDB0 > 2) ? kDB0 / 2 : kDB0);
  constexpr int kDB = kDB1 * CPT > 128 ? 128 / CPT : kDB1;
  constexpr int UB = 8;                  // predictor-row vectors per lane per batch
  // up-row vectors per lane per batch, two batches in flight: 8 (4 for the
  // short INT4 rows), halved for ReGLU's second row and for 4+ tokens
  constexpr int UBU0 = (WT == WT_I4 ? 4 : 8) / (ACT == ACT_REGLU ? 2 : 1) / (NT >= 4 ? 2 : 1);
  constexpr int UBU = UBU0 < 2 ? 2 : UBU0;
  constexpr int SP = NT == 2 ? 8 : 4;    // staged x vectors per thread held in registers
  extern __shared__ __align__(16) unsigned char smem[];
  XT* xs = reinterpret_cast<XT*>(smem);
  __shared__ int s_idw[NW][kMaxPer];     // each wavefront's copy of the run's neuron ids
  __shared__ float s_h[NT][kMaxPer];
  __shared__ float s_red[NT][16];

  const int d = a.d, f = a.f;
  const int G = vg, g = vb;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  int* ids_w = s_idw[wave];
  const int row_bytes = (WT == WT_F32) ? d * 4 : (WT == WT_F16 ? d * 2 : d / 2);
  const int nvec = row_bytes / 16;
  const int ngroups = d / 128;
  const int words = f / 64;
  const int col0 = threadIdx.x * CPT;
  const bool colok = col0 < d;
  const int col = colok ? col0 : 0;  // keeps every address in bounds

  // ---- 1. loads that wait for nothing: the mask words (lane-major: lane l
  // of every wavefront holds words l*UW .. l*UW + UW-1, read in 16-byte
  // pairs), the layer input, the first batch of this wavefront's predictor
  // row.  The guarded loads come first; the weight loads after them are
  // unconditional, so later waits can skip those.
  static_assert(UW % 2 == 0, "mask words are read in pairs");
  uint64_t u[SRC == SRC_UNION ? UW : 1];
  if constexpr (SRC == SRC_UNION) {
#pragma unroll
    for (int k = 0; k < UW; k += 2) {
      const int w = lane * UW + k;
      u[k] = u[k + 1] = 0ull;
      if (w + 1 < words) {
        const u32x4 q = *reinterpret_cast<const u32x4*>(a.union_mask + w);
        u[k] = ((uint64_t)q.y << 32) | q.x;
        u[k + 1] = ((uint64_t)q.w << 32) | q.z;
      } else if (w < words) {
        u[k] = a.union_mask[w];
      }
    }
  }
  int n_ids = 0;
  if constexpr (SRC == SRC_IDS) n_ids = *a.count;
  StageSplit<XT, WT == WT_I4, SP> stage;
  constexpr int CV = CHAIN ? ffn_chain_vecs(NT, CPT) : 1;
  f32x4 rv[CV];
  if constexpr (CHAIN)
    chain_issue<NT, CV, true>(a.r_in, rv, d, a.tok0, a.nt);  // CV is sized to the shape
  else
    stage.issue(reinterpret_cast<const XT*>(a.x), d, a.tok0, a.nt, NT);

  constexpr int PWT = WT == WT_F32 ? WT_F32 : WT_F16;
  const int pr = P1 ? (a.r + G - 1) / G : 0;
  const int p0 = g * pr;
  const int pnvec = d * (int)sizeof(XT) / 16;
  const int pk0 = NW - 1 - wave;  // this wavefront's first predictor row (local)
  RowLoads<PWT, kWave, UB> Lp;
  if constexpr (P1) {
    // a wavefront without a predictor row reads one shared vector of the
    // mask instead (w1_t is null when there is no next layer)
    const bool have = pk0 < pr && p0 + pk0 < a.r;
    const uint8_t* prow = have ? a.w1_t + (size_t)(p0 + pk0) * d * sizeof(XT)
                               : reinterpret_cast<const uint8_t*>(a.union_mask);
    Lp.issue(prow, nullptr, have ? pnvec : 1, (have && lane < pnvec) ? lane : 0);
  }

  // ---- 2. the run [s0, s1) of active slots and its neuron ids ----------------
  int cnt;
  if constexpr (SRC == SRC_UNION) {
    int c = 0;
#pragma unroll
    for (int k = 0; k < UW; ++k) c += __popcll(u[k]);
    const int incl = wave_incl_scan(c);
    const int total = __builtin_amdgcn_readlane(incl, kWave - 1);
    const int ex = incl - c;  // slots before this lane's words
    const int per = (total + G - 1) / G;
    const int s0 = g * per;
    const int s1 = (s0 + per < total) ? s0 + per : total;
    cnt = s1 > s0 ? s1 - s0 : 0;
    const bool wr = a.write_ids && wave == 0;
    if (cnt > 0) {
      // from the lane whose words hold slot s0, walk the words in order (scalar
      // counts); each word holding slots of the run is emitted by the 64 lanes
      // together, lane b taking bit b
      int L = __builtin_ctzll(__ballot(ex + c > s0));
      int off = __builtin_amdgcn_readlane(ex, L);
      while (off < s1 && L < kWave) {
#pragma unroll
        for (int k = 0; k < UW; ++k) {
          if (off < s1) {
            const uint64_t word = readlane64(u[k], L);
            const int pw = __popcll(word);
            if (off + pw > s0) {
              const int slot = off + bits_below_lane(word);
              if (((word >> lane) & 1ull) && slot >= s0 && slot < s1) {
                const int id = (L * UW + k) * 64 + lane;
                ids_w[slot - s0] = id;
                if (wr) a.ids_out[slot] = id;
              }
            }
            off += pw;
          }
        }
        ++L;
      }
    }
    if (a.write_ids && g == 0 && threadIdx.x == 0) *a.count_out = total;
  } else {
    int n = f;
    if constexpr (SRC == SRC_IDS) n = n_ids < 0 ? 0 : (n_ids > f ? f : n_ids);
    const int per = (n + G - 1) / G;
    const int s0 = g * per;
    cnt = (s0 + per < n) ? per : (n > s0 ? n - s0 : 0);
    for (int j = lane; j < cnt; j += kWave) {
      const int id = (SRC == SRC_IDS) ? a.ids[s0 + j] : s0 + j;
      ids_w[j] = ((unsigned)id < (unsigned)f) ? id : -1;
    }
  }
  __builtin_amdgcn_wave_barrier();  // the wavefront's list is written before any lane reads it

  // ---- 3. first weight loads, before x is ready: this wavefront's first up
  // (+ gate) batch and the first batch of W_down^T rows --------------------
  RowLoads<WT, kWave, UBU> Lu, Lg;
  {
    const int i = wave < cnt ? ids_w[wave] : -1;
    const bool have = i >= 0;  // else one shared vector of row 0
    const size_t ro = have ? (size_t)i * row_bytes : 0;
    const size_t so = have ? (size_t)i * ngroups : 0;
    const int n0 = have ? nvec : 1;
    const int v0 = (have && lane < nvec) ? lane : 0;
    Lu.issue(a.w_up + ro, a.s_up ? a.s_up + so : nullptr, n0, v0);
    if constexpr (ACT == ACT_REGLU) Lg.issue(a.w_gate + ro, a.s_gate ? a.s_gate + so : nullptr, n0, v0);
  }
  DownCols<WT, CPT> wd[2][kDB];
#pragma unroll
  for (int u2 = 0; u2 < kDB; ++u2) {
    const int iu = u2 < cnt ? ids_w[u2] : (cnt > 0 ? ids_w[0] : 0);
    wd[0][u2].load(a.w_down_t, a.s_down_t, iu >= 0 ? iu : 0, col, d);
  }
  __builtin_amdgcn_sched_barrier(0);  // every load above is issued before the staging waits

  // ---- 4. x into LDS: staged activations, or the residual chain -------------
  if constexpr (CHAIN)
    chain_finish<XT, NT, WT == WT_I4, CV>(rv, xs, s_red, a.x_out, g == 0, a.eps, d, a.tok0, a.nt);
  else
    stage.commit(xs, reinterpret_cast<const XT*>(a.x), d, a.tok0, a.nt, NT);
  __syncthreads();

  // ---- 5. up (+ gate) rows: one wavefront per slot -------------------------
  // The wavefront's rows (slots wave, wave + NW, ...) are walked as one
  // sequence of batches of UBU vectors per lane, two buffers deep: batch q+1
  // (of this row or the next) is requested before batch q is used, so a
  // wavefront with many rows keeps a row in flight while it computes.
  {
    const int bstep = UBU * kWave;
    const int nb = (nvec + bstep - 1) / bstep;                    // batches per row
    const int nrow = wave < cnt ? (cnt - 1 - wave) / NW + 1 : 0;  // this wavefront's rows
    const int nq = nrow * nb;
    RowLoads<WT, kWave, UBU> Lu2, Lg2;  // Lu / Lg hold batch 0 (step 3)
    int pk = 0, pb = 0;                 // row and batch of the last request
    int ck = 0, cb = 0;                 // row and batch being used
    float au[NT], ag[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) au[t] = ag[t] = 0.0f;
    for (int q = 0; q < nq; q += 2) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        if (q + hb < nq) {  // wave-uniform
          RowLoads<WT, kWave, UBU>& Lc = hb ? Lu2 : Lu;
          RowLoads<WT, kWave, UBU>& Ln = hb ? Lu : Lu2;
          RowLoads<WT, kWave, UBU>& Gc = hb ? Lg2 : Lg;
          RowLoads<WT, kWave, UBU>& Gn = hb ? Lg : Lg2;
          if (q + hb + 1 < nq) {  // request the next batch into the other buffer
            if (++pb == nb) {
              pb = 0;
              ++pk;
            }
            const int in = ids_w[wave + pk * NW];
            const int inc = in >= 0 ? in : 0;
            const int v0 = lane + pb * bstep;
            const int v0c = v0 < nvec ? v0 : 0;  // lanes past a short row read its first vector
            Ln.issue(a.w_up + (size_t)inc * row_bytes, a.s_up ? a.s_up + (size_t)inc * ngroups : nullptr, nvec,
                     v0c);
            if constexpr (ACT == ACT_REGLU)
              Gn.issue(a.w_gate + (size_t)inc * row_bytes, a.s_gate ? a.s_gate + (size_t)inc * ngroups : nullptr,
                       nvec, v0c);
          }
          __builtin_amdgcn_sched_barrier(0);  // the next batch is requested before this one is used
          const int v0 = lane + cb * bstep;
          Lc.template consume<NT>(nvec, v0, xs, d, au);
          if constexpr (ACT == ACT_REGLU) Gc.template consume<NT>(nvec, v0, xs, d, ag);
          if (++cb == nb) {  // the row is done: h for its slot
            const int j = wave + ck * NW;
            const int i = ids_w[j];
            const bool ok = i >= 0;
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
#pragma unroll
            for (int t = 0; t < NT; ++t) au[t] = ag[t] = 0.0f;
            cb = 0;
            ++ck;
          }
        }
      }
    }
  }
  if constexpr (P1) {
    // z[t][row] = W1^T[row] . x[t]; x is staged in the INT4 pairing order when
    // the FFN is INT4, so W1's fp16 vectors are paired the same way
    for (int k = pk0; k < pr && p0 + k < a.r; k += NW) {  // wave-uniform
      const uint8_t* prow = a.w1_t + (size_t)(p0 + k) * d * sizeof(XT);
      float acc[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t] = 0.0f;
      for (int v0 = lane; v0 < pnvec; v0 += UB * kWave) {
        if (!(k == pk0 && v0 == lane)) Lp.issue(prow, nullptr, pnvec, v0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < UB; ++u) {
          const int v = v0 + u * kWave;
          const bool ok = v < pnvec;
          const int vc = ok ? v : 0;
          u32x4 wv = ok ? Lp.w[u] : u32x4{0u, 0u, 0u, 0u};
          if constexpr (WT == WT_F32) {
            vec_f32<NT>(wv, reinterpret_cast<const float*>(xs) + 4 * vc, d, acc);
          } else {
            if constexpr (WT == WT_I4) wv = StageSplit<XT, true, 1>::perm8(wv);
            vec_f16<NT>(wv, reinterpret_cast<const f16*>(xs) + 8 * vc, d, acc);
          }
        }
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t] = group_sum<kWave>(acc[t]);
      if (lane == 0) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
          if (t < a.nt) a.z[(size_t)(a.tok0 + t) * a.r + p0 + k] = acc[t];
      }
    }
  }
  __syncthreads();

  // ---- 6. down: acc[t][k] += h[t][j] * W_down^T[id_j][col + k], slots in order
  // INT4: acc[t][k] += (h[t][j] * s_j) * (q_jk + 8) with q + 8 read straight
  // from the offset-binary nibble as a byte; the 8 * sum_j h s_j that this adds
  // to every column is taken off at the end (sb).
  float acc[NT][CPT];
  float sb[WT == WT_I4 ? NT : 1];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int k = 0; k < CPT; ++k) acc[t][k] = 0.0f;
    if constexpr (WT == WT_I4) sb[t] = 0.0f;
  }

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
            const int iu = ids_w[jj];
            wd[half ^ 1][u].load(a.w_down_t, a.s_down_t, iu >= 0 ? iu : 0, col, d);
          }
        }
#pragma unroll
        for (int u = 0; u < kDB; ++u) {
          const int jj = jb + u;
          const int jc = jj < cnt ? jj : jb;
          const bool ok = jj < cnt && ids_w[jc] >= 0 && colok;
          if constexpr (WT == WT_I4) {
            float hs[NT];
#pragma unroll
            for (int t = 0; t < NT; ++t) {
              hs[t] = ok ? s_h[t][jc] * wd[half][u].s : 0.0f;  // a select: a poisoned scale never enters
              sb[t] += hs[t];
            }
#pragma unroll
            for (int m = 0; m < CPT / 8; ++m) {
              const uint32_t v = wd[half][u].q[m] ^ 0x88888888u;  // nibbles as q + 8
              const uint32_t lo = v & 0x0F0F0F0Fu, hi = (v >> 4) & 0x0F0F0F0Fu;
              float n[8];
#pragma unroll
              for (int b = 0; b < 4; ++b) {
                n[2 * b] = (float)((lo >> (8 * b)) & 0xFFu);
                n[2 * b + 1] = (float)((hi >> (8 * b)) & 0xFFu);
              }
#pragma unroll
              for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int k = 0; k < 8; ++k) acc[t][8 * m + k] = __builtin_fmaf(hs[t], n[k], acc[t][8 * m + k]);
            }
          } else {
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
  }

  if constexpr (WT == WT_I4) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int k = 0; k < CPT; ++k) acc[t][k] = __builtin_fmaf(-8.0f, sb[t], acc[t][k]);
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

struct SumArgs {
  const float* partial;  // [G][B][d]
  int G, B, d, xtype;
  const void* b_down;    // [d] in x's type, or null
  float* y;              // [B][d] or null
  const float* r_in;     // residual add: r_out = r_in + y (null to skip)
  float* r_out;
};

// y[e] = b_down[c] + sum over workgroups g = 0..G-1 of partial[g][e], e = t*d + c.
// A 512-thread workgroup covers kSumEPW elements: thread (q, c) adds the
// partials of g-group q (of kSumNQ, kSumBat consecutive g's) in order, then
// the group sums are added in order.  Split in two so that a fused launch can
// issue these loads, do other work, and finish the sum afterwards.  Requires
// G <= kSumNQ * kSumBat.
constexpr int kSumEPW = 16;
constexpr int kSumNQ = 512 / kSumEPW;
constexpr int kSumBat = 16;

// Element block of sum workgroup vb: workgroups are dealt to the 8 XCDs in
// turn (vb % 8), so blocks 2m and 2m+1, which share each 128-byte line of
// the partials, go to workgroups vb and vb + 8 of one XCD and the line is
// fetched into that XCD's L2 once.
__device__ __forceinline__ int sum_block(int vb, int gs) {
  if (vb >= (gs & ~15)) return vb;
  return (vb & ~15) + 2 * (vb & 7) + ((vb >> 3) & 1);
}

struct SumLoads {
  float p[kSumBat];
  float bias, rin;  // this element's b_down and residual, fetched with the partials
};

__device__ __forceinline__ void sum_issue(const SumArgs& a, int vb, int gs, SumLoads& L) {
  const int c16 = threadIdx.x % kSumEPW, q = threadIdx.x / kSumEPW;
  const int n = a.B * a.d;
  const int e = sum_block(vb, gs) * kSumEPW + c16;
  const int ec = e < n ? e : 0;
  const int per = (a.G + kSumNQ - 1) / kSumNQ;
  const int g0 = q * per;
#pragma unroll
  for (int j = 0; j < kSumBat; ++j) {
    L.p[j] = 0.0f;
    if (j < per && g0 + j < a.G) L.p[j] = a.partial[(size_t)(g0 + j) * n + ec];
  }
  L.bias = 0.0f;
  L.rin = 0.0f;
  if (q == 0) {
    const int c = ec % a.d;
    if (a.b_down) L.bias = (a.xtype == WT_F32) ? load_as_float<float>(a.b_down, c) : load_as_float<f16>(a.b_down, c);
    if (a.r_in) L.rin = a.r_in[ec];
  }
}

__device__ __forceinline__ void sum_finish(const SumArgs& a, int vb, int gs, const SumLoads& L) {
  __shared__ float part[kSumNQ][kSumEPW];
  const int c16 = threadIdx.x % kSumEPW, q = threadIdx.x / kSumEPW;
  const int n = a.B * a.d;
  const int e = sum_block(vb, gs) * kSumEPW + c16;
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < kSumBat; ++j) s += L.p[j];  // slots past the group hold zeros
  part[q][c16] = s;
  __syncthreads();
  if (q == 0 && e < n) {
    float tot = 0.0f;
#pragma unroll
    for (int k = 0; k < kSumNQ; ++k) tot += part[k][c16];
    const float v = L.bias + tot;
    if (a.y) a.y[e] = v;
    if (a.r_in) a.r_out[e] = L.rin + v;
  }
}

__device__ __forceinline__ void sum_body(const SumArgs& a, int vb, int gs) {
  SumLoads L;
  sum_issue(a, vb, gs, L);
  sum_finish(a, vb, gs, L);
}

// Shape choices and argument builders shared by the launchers.
struct FfnShape {
  int cpt, nth, nt;
};
FfnShape ffn_shape(int wt, int d, int batch);
FfnArgs ffn_args(const FfnLaunch& p, int tok0, int nt, bool first);
SumArgs sum_args(const FfnLaunch& p);
int sum_groups(int batch, int d);

}  // namespace sfnn
