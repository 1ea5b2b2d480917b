// Up-projection body of the neuron-gathered FFN: only the listed neurons'
// rows are read.
//
// A zero activation zeroes the whole row of the down projection it multiplies,
// so that row need not be loaded at all (53ai.com sparsity survey, section
// 激活稀疏); PowerInfer's GPU operators work on individual neuron rows and
// columns (same survey, PowerInfer 概述).  Storage is neuron-major: neuron i
// owns row i of W_up, W_gate and W_down^T, each a contiguous d_model run.
//
// up_body: one workgroup computes the activations of a contiguous run of the
//   active slots:
//   1. the run and its neuron ids come from the caller's list, from the
//      identity (dense), or from compacting the union mask in the prologue
//      (popcounts + a lane prefix sum over all mask words in every
//      wavefront; no separate compaction launch between the predictor and
//      the FFN);
//   2. up (+ gate): one wavefront per neuron row, 16-byte coalesced loads,
//      activations in LDS, ReLU / ReGLU and the per-token select fused;
//   3. h[t][slot] goes to global memory (and the run's ids, when compacting),
//      for the column-tiled down projection of the next launch
//      (down_body.hpp), which writes y without partial rows.
// The body takes a virtual workgroup index so that a launch can run it beside
// other work (the look-ahead stack adds the next layer's predictor rows).
#pragma once
#include "common.hpp"
#include "launch.hpp"
#include "pred_body.hpp"

namespace sfnn {

constexpr int kMaxPer = 512;  // slots one FFN workgroup can own

// Up-row batches a wavefront keeps in flight (2 to 4).
#ifndef SFNN_UP_NBUF
#define SFNN_UP_NBUF 2
#endif
template <int WT, int NT>
constexpr int up_nbuf() { return SFNN_UP_NBUF; }

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
  float* hout;           // h [B][hstride] fp32, slot order
  int hstride;
  const float* r_in;     // residual rows (chain prologue: x = r / rms(r)) or null
  void* x_out;           // chain prologue: x written here by workgroup 0 (or null)
  float eps;
  const uint8_t* w1_t;   // p1_body: the next layer's predictor W1^T [r][d] (stage 1 on the same x)
  float* z;              // p1_body: its output [B][r]
  int r;                 // p1_body: rank
  int d, f, B, tok0, nt, write_ids;
};

// One batch of an up (+ gate) row in flight: the weight vectors, and the
// row's bias and per-token mask word, requested with them so that finishing
// a row needs no load of its own (a load in a branch there would make the
// next wait cover every load in flight, the next batch's included).
template <int WT, int UBU>
struct UpBatch {
  RowLoads<WT, kWave, UBU> u, g;
  float bu, bg;  // b_up[i], b_gate[i] (0 without biases)
  uint64_t mw;   // mask word of neuron i for this lane's token (all ones without a gate)
  int i;         // neuron id (< 0: a slot that adds nothing)
};

// One up-projection workgroup (virtual index vb of vg).  CHAIN: the layer input is
// x = r_in / rms(r_in), built in the prologue instead of staged from a.x.
// Every wavefront derives the workgroup's slot list by itself (mask words,
// popcounts, one lane scan, then the 64 bits of each word that holds slots
// of the run emitted by the 64 lanes at once into the wavefront's own LDS
// list), so no workgroup barrier stands between the mask and the first
// weight loads: the barriers that stage x come after those loads are issued.
// RV: float4 vectors per thread per token of the residual row (CHAIN only;
// d_model <= 4 RV NTH).
template <int WT, int ACT, int NT, int SRC, int NTH, int RV, bool CHAIN, int UW>
__device__ __forceinline__ void up_body(const FfnArgs& a, int vb, int vg) {
  using XT = typename std::conditional<WT == WT_F32, float, f16>::type;
  constexpr int NW = NTH / kWave;
  // up-row vectors per lane per batch, two batches in flight: 8 (4 for the
  // INT4 rows from two tokens on), halved for ReGLU's second row and for 4+
  // tokens
  constexpr int UBU0 = (WT == WT_I4 && NT > 1 ? 4 : 8) / (ACT == ACT_REGLU ? 2 : 1) / (NT >= 4 ? 2 : 1);
  constexpr int UBU = UBU0 < 2 ? 2 : UBU0;
  constexpr int NBUF = up_nbuf<WT, NT>();
  constexpr int SP = NT == 2 ? 8 : 4;    // staged x vectors per thread held in registers
  extern __shared__ __align__(16) unsigned char smem[];
  XT* xs = reinterpret_cast<XT*>(smem);
  // INT4: -8 times the sum of each 32 staged activations, [NT][d / 32], behind xs
  float* m8 = reinterpret_cast<float*>(smem + (size_t)NT * a.d * sizeof(XT));
  __shared__ int s_idw[NW][kMaxPer];     // each wavefront's copy of the run's neuron ids
  __shared__ float s_red[NT][16];

  const int d = a.d, f = a.f;
  const int G = vg, g = vb;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform, in a scalar register
  int* ids_w = s_idw[wave];
  const int row_bytes = (WT == WT_F32) ? d * 4 : (WT == WT_F16 ? d * 2 : d / 2);
  const int nvec = row_bytes / 16;
  const int ngroups = d / 128;
  const int words = f / 64;

  // ---- 1. loads that wait for nothing: the mask words (lane-major: lane l
  // of every wavefront holds words l*UW .. l*UW + UW-1, read in 16-byte
  // pairs) and the layer input.  The guarded loads come first; the weight
  // loads after them are unconditional, so later waits can skip those.
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
  constexpr int CV = CHAIN ? NT * RV : 1;
  f32x4 rv[CV];
  if constexpr (CHAIN)
    chain_issue<NT, CV, true>(a.r_in, rv, d, a.tok0, a.nt);  // CV is sized to the shape
  else
    stage.issue(reinterpret_cast<const XT*>(a.x), d, a.tok0, a.nt, NT);

  // ---- 2. the run [s0, s0 + cnt) of active slots and its neuron ids --------
  int cnt, s0;
  if constexpr (SRC == SRC_UNION) {
    int c = 0;
#pragma unroll
    for (int k = 0; k < UW; ++k) c += __popcll(u[k]);
    const int incl = wave_incl_scan(c);
    const int total = __builtin_amdgcn_readlane(incl, kWave - 1);
    const int ex = incl - c;  // slots before this lane's words
    const int per = (total + G - 1) / G;
    s0 = g * per;
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
    s0 = g * per;
    cnt = (s0 + per < n) ? per : (n > s0 ? n - s0 : 0);
    for (int j = lane; j < cnt; j += kWave) {
      const int id = (SRC == SRC_IDS) ? a.ids[s0 + j] : s0 + j;
      ids_w[j] = ((unsigned)id < (unsigned)f) ? id : -1;
    }
  }
  __builtin_amdgcn_wave_barrier();  // the wavefront's list is written before any lane reads it

  // ---- 3. first weight loads, before x is ready: this wavefront's first up
  // (+ gate) batch ------------------------------------------------------------
  // Batch (k, pb) of this wavefront: batch pb of its k-th row (slot
  // wave + k NW).  Every load is unconditional: a slot past the run (or an
  // invalid id) reads row 0's vectors and adds nothing; a missing bias or
  // gate reads element 0 of x instead and is not used.
  const int bstep = UBU * kWave;
  const int tt = lane < a.nt ? lane : 0;  // the token this lane finishes (lanes >= nt repeat token 0)
  auto up_issue = [&](UpBatch<WT, UBU>& Bt, int k, int pb) {
    const int j = wave + k * NW;
    const int i = j < cnt ? ids_w[j < kMaxPer ? j : 0] : -1;
    const bool have = i >= 0;
    const int inc = have ? i : 0;
    const int v0 = lane + pb * bstep;
    const int v0c = (have && v0 < nvec) ? v0 : 0;  // lanes past a short row read its first vector
    Bt.i = i;
    // the small loads first: a wait for them then never covers this batch's
    // weight loads
    const uint64_t* msrc = a.mask ? a.mask + (size_t)(a.tok0 + tt) * words + (inc >> 6)
                                  : reinterpret_cast<const uint64_t*>(a.x);
    Bt.mw = *msrc;
    const void* bsu = a.b_up ? a.b_up : a.x;
    Bt.bu = load_as_float<XT>(bsu, a.b_up ? inc : 0);
    if constexpr (ACT == ACT_REGLU) {
      const void* bsg = a.b_gate ? a.b_gate : a.x;
      Bt.bg = load_as_float<XT>(bsg, a.b_gate ? inc : 0);
    }
    Bt.u.issue(a.w_up + (size_t)inc * row_bytes, a.s_up ? a.s_up + (size_t)inc * ngroups : nullptr,
               have ? nvec : 1, v0c);
    if constexpr (ACT == ACT_REGLU)
      Bt.g.issue(a.w_gate + (size_t)inc * row_bytes, a.s_gate ? a.s_gate + (size_t)inc * ngroups : nullptr,
                 have ? nvec : 1, v0c);
  };
  // this wavefront's rows and batches (wave-uniform: scalar loop control)
  const int nb = (nvec + bstep - 1) / bstep;  // batches per row
  const int nrow = __builtin_amdgcn_readfirstlane(wave < cnt ? (cnt - 1 - wave) / NW + 1 : 0);
  const int nq = nrow * nb;
  int pk = 0, pb = 0;  // row and batch of the last request
  // request the batch after the last one (past the end: the last batch again)
  auto up_next = [&](UpBatch<WT, UBU>& Bn) {
    if (++pb == nb) {
      pb = 0;
      ++pk;
    }
    const bool past = pk >= nrow;
    up_issue(Bn, past ? (nrow > 0 ? nrow - 1 : 0) : pk, past ? nb - 1 : pb);
  };
  UpBatch<WT, UBU> Bq[NBUF];
  up_issue(Bq[0], 0, 0);
#pragma unroll
  for (int j = 1; j < NBUF - 1; ++j) up_next(Bq[j]);
  __builtin_amdgcn_sched_barrier(0);  // every load above is issued before the staging waits
  // in the look-ahead launch the prologue up to here ran at a raised wave
  // priority; the rest runs at the stage-1 workgroups' level or just above
  if constexpr (CHAIN) __builtin_amdgcn_s_setprio(1);

  // ---- 4. x into LDS: staged activations, or the residual chain -------------
  if constexpr (CHAIN)
    chain_finish<XT, NT, WT == WT_I4, CV>(rv, xs, s_red, a.x_out, g == 0, a.eps, d, a.tok0, a.nt);
  else
    stage.commit(xs, reinterpret_cast<const XT*>(a.x), d, a.tok0, a.nt, NT);
  __syncthreads();
  if constexpr (WT == WT_I4) {
    // the offset's share of every 32-element vector (vec_i4), once per token
    const int nv = d / 32;
    for (int i = threadIdx.x; i < NT * nv; i += NTH) {
      const f16* xp = reinterpret_cast<const f16*>(xs) + (size_t)(i / nv) * d + 32 * (i % nv);
      float sx = 0.0f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const u32x4 q = *reinterpret_cast<const u32x4*>(xp + 8 * k);
        const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const f16x2 h2 = bitcast<f16x2>(u[m]);
          sx += (float)h2.x;
          sx += (float)h2.y;
        }
      }
      m8[i] = -8.0f * sx;
    }
    __syncthreads();
  }

  // ---- 5. up (+ gate) rows: one wavefront per slot -------------------------
  // The wavefront's rows (slots wave, wave + NW, ...) are walked as one
  // sequence of batches of UBU vectors per lane, NBUF buffers deep: batches
  // q+1 .. q+NBUF-1 (of this row or the next) are requested before batch q is
  // used, so a wavefront keeps rows in flight while it computes.  The loop
  // leaves by break and requests harmless repeats of the last batch at the
  // end, so no load and no store sits in a branch.
  {
    int ck = 0, cb = 0;  // row and batch being used
    float au[NT], ag[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) au[t] = ag[t] = 0.0f;
    auto up_step = [&](UpBatch<WT, UBU>& Bc, UpBatch<WT, UBU>& Bn) {
      up_next(Bn);  // into the buffer used last
      __builtin_amdgcn_sched_barrier(0);  // the next batch is requested before this one is used
      const int v0 = lane + cb * bstep;
      const int vb = cb * bstep;  // lane 0's v0 (wave-uniform)
      Bc.u.template consume<NT>(nvec, v0, xs, d, au, m8, d / 32, vb);
      if constexpr (ACT == ACT_REGLU) Bc.g.template consume<NT>(nvec, v0, xs, d, ag, m8, d / 32, vb);
      if (++cb == nb) {  // the row is done: h for its slot
        const int j = wave + ck * NW;
        const int i = Bc.i;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          au[t] = group_sum<kWave>(au[t]);
          if (ACT == ACT_REGLU) ag[t] = group_sum<kWave>(ag[t]);
        }
        // lane l finishes token tt (every lane stores; lanes >= nt repeat
        // token 0's value at its address)
        float ut = 0.0f, gt = 0.0f;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          ut = tt == t ? au[t] : ut;
          gt = tt == t ? ag[t] : gt;
        }
        const float up = ut + (a.b_up ? Bc.bu : 0.0f);
        float hv;
        if constexpr (ACT == ACT_RELU) {
          hv = up > 0.0f ? up : 0.0f;
        } else {
          const float g = gt + (a.b_gate ? Bc.bg : 0.0f);
          hv = (g > 0.0f ? g : 0.0f) * up;
        }
        const bool on = !a.mask || ((Bc.mw >> (i & 63)) & 1ull);  // select: gated-off neurons add nothing
        hv = (i >= 0 && on) ? hv : 0.0f;
        a.hout[(size_t)(a.tok0 + tt) * a.hstride + s0 + j] = hv;
#pragma unroll
        for (int t = 0; t < NT; ++t) au[t] = ag[t] = 0.0f;
        cb = 0;
        ++ck;
      }
    };
    if (nq > 0) {  // wave-uniform
      for (int q = 0;; q += NBUF) {
        up_step(Bq[0], Bq[NBUF - 1]);
        if (q + 1 >= nq) break;
        up_step(Bq[1], Bq[0]);
        if (q + 2 >= nq) break;
        if constexpr (NBUF >= 3) {
          up_step(Bq[2], Bq[1]);
          if (q + 3 >= nq) break;
        }
        if constexpr (NBUF >= 4) {
          up_step(Bq[3], Bq[2]);
          if (q + 4 >= nq) break;
        }
      }
    }
  }
}

// Predictor stage 1 of the next layer for virtual workgroup vb of vg (the
// look-ahead stack's launch A runs these beside the up-projection
// workgroups, on the same layer input): z[t][p0 + k] = W1^T[p0 + k] . x[t]
// for this workgroup's rows [p0, p0 + pr).  x = r_in / rms(r_in) is built in
// the prologue, as in up_body.  Each row is split in NW equal column chunks,
// one per wavefront, so every wavefront carries the same share; a pass of PR
// rows has all its loads in flight at once (issued before the prologue
// waits), and the wavefronts' partial dots are added in LDS in wavefront
// order.  RV as in up_body.  LATE: the first pass of W1^T rows is requested
// only once x is built.  The up workgroups that share the CUs then get their
// mask words and first up rows through the memory pipeline before the W1
// stream fills it; worth it where their prologue is long (INT4 rows with
// their scales: OPT-175B layer 47.1 -> 45.2 us; at fp16 OPT-6.7B it costs 5%).
template <int WT, int NT, int NTH, int RV, bool LATE = false>
__device__ __forceinline__ void p1_body(const FfnArgs& a, int vb, int vg) {
  using XT = typename std::conditional<WT == WT_F32, float, f16>::type;
  constexpr int NW = NTH / kWave;
  constexpr int PV = (WT == WT_F32 ? 2 : 1) * RV / 2;  // PV * 64 * NW vectors cover d_model <= 4 RV NTH
  constexpr int PR = PV <= 2 ? 8 : 4;
  extern __shared__ __align__(16) unsigned char smem[];
  XT* xs = reinterpret_cast<XT*>(smem);
  __shared__ float s_red[NT][16];
  __shared__ float s_pz[NT][PR][NW];
  const int d = a.d;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int pr = (a.r + vg - 1) / vg;
  const int p0 = vb * pr;
  const int pcw = d * (int)sizeof(XT) / 16 / NW;  // vectors per wavefront chunk of a row
  constexpr int CV = NT * RV;
  f32x4 rv[CV];
  chain_issue<NT, CV, true>(a.r_in, rv, d, a.tok0, a.nt);
  u32x4 pw[PR][PV];
  // one pass of rows (k0 .. k0 + PR - 1 of this workgroup's); a row past the
  // share or the rank reads row 0's vectors and is not written
  auto issue = [&](int k0) {
#pragma unroll
    for (int k = 0; k < PR; ++k) {
      const int j = p0 + k0 + k;
      const bool have = k0 + k < pr && j < a.r;
      const uint8_t* prow = a.w1_t + (size_t)(have ? j : 0) * d * sizeof(XT);
#pragma unroll
      for (int v = 0; v < PV; ++v) {
        const int vi = lane + kWave * v;
        pw[k][v] = ld16_stream(prow + 16 * (size_t)(wave * pcw + (vi < pcw ? vi : 0)));
      }
    }
  };
  if constexpr (!LATE) issue(0);
  __builtin_amdgcn_sched_barrier(0);  // every load above is issued before the prologue waits
  chain_finish<XT, NT, false, CV>(rv, xs, s_red, nullptr, false, a.eps, d, a.tok0, a.nt);
  __syncthreads();
  for (int k0 = 0; k0 < pr; k0 += PR) {  // workgroup-uniform
    if (k0 > 0 || LATE) issue(k0);
    float pacc[PR][NT];
#pragma unroll
    for (int k = 0; k < PR; ++k) {
#pragma unroll
      for (int t = 0; t < NT; ++t) pacc[k][t] = 0.0f;
#pragma unroll
      for (int v = 0; v < PV; ++v) {
        const int vi = lane + kWave * v;
        const bool ok = vi < pcw;
        const int vc = ok ? wave * pcw + vi : 0;
        const u32x4 wv = ok ? pw[k][v] : u32x4{0u, 0u, 0u, 0u};
        if constexpr (WT == WT_F32)
          vec_f32<NT>(wv, reinterpret_cast<const float*>(xs) + 4 * vc, d, pacc[k]);
        else
          vec_f16<NT>(wv, reinterpret_cast<const f16*>(xs) + 8 * vc, d, pacc[k]);
      }
    }
#pragma unroll
    for (int k = 0; k < PR; ++k)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float sw = wave_sum(pacc[k][t]);
        if (lane == 0) s_pz[t][k][wave] = sw;
      }
    __syncthreads();
    if ((int)threadIdx.x < NT * PR) {
      const int t = threadIdx.x / PR, k = threadIdx.x % PR;
      float z = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) z += s_pz[t][k][w];
      if (t < a.nt && k0 + k < pr && p0 + k0 + k < a.r) a.z[(size_t)(a.tok0 + t) * a.r + p0 + k0 + k] = z;
    }
    __syncthreads();  // s_pz is reused by the next pass
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
  int rv, nth, nt;  // residual float4 vectors per thread per token, threads, tokens per pass
};
FfnShape ffn_shape(int wt, int d, int batch);
FfnArgs ffn_args(const FfnLaunch& p, int tok0, int nt, bool first);
SumArgs sum_args(const FfnLaunch& p, int rows);  // rows: partial rows per token
hipError_t launch_sum_args(const SumArgs& a, hipStream_t s);
int sum_groups(int batch, int d);

}  // namespace sfnn
