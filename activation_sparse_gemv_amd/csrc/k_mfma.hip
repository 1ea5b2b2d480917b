// Larger batches of the gathered FFN on the matrix cores (fp16 weights).
//
// Once a batch has a dozen tokens the FFN over its union of active neurons is
// a dense contraction: h = act(W_up[U] x^T) over |U| gathered rows and
// y = W_down^T[U]^T h over the same rows (PowerInfer's neuron-aware operators,
// [53ai] GPU-CPU混合执行; the per-row work of the pages, batched).  The VALU
// kernels re-read the weights once per token group at such batches; here one
// pass covers up to 32 tokens with v_mfma_f32_16x16x32_f16, fp32 accumulation.
//
//  k_up_mfma   workgroup = 32 gathered rows (two 16-row tiles); its 8
//              wavefronts split d_model into 64-column pairs (wavefront w
//              takes pairs w, w+8, ...), each holding a 16x16 fp32 block per
//              (tile, 16 tokens); the blocks are added in wavefront order in
//              LDS, then bias, activation and the per-token select give
//              h [token][slot] in fp32, and the largest |h| of each token
//              over the workgroup's 32 slots.
//  k_down_mfma workgroup = 128 (one token tile) or 64 (two) output columns
//              x one group of slots; its 8
//              wavefronts split the group's 32-slot steps.  Each token's h is
//              scaled by a power of two chosen from its largest |h| over the
//              group's slots and split into two fp16 planes hi + lo (hi =
//              fp16(h), lo = fp16(h - hi): 22 of fp32's 24 significant bits,
//              exact for integers below 2^22, no overflow at any |h|); both
//              planes are multiplied and the product scaled back.  One fp32
//              partial row per group and token, added in a fixed order by
//              k_sum.
//
// MFMA operands (16x16x32): lane l holds 8 consecutive K values of row
// l % 16 of A and of column l % 16 of B, K block l / 16; D row 4*(l/16) + q,
// column l % 16 in register q.  Up: A = 16 weight rows (contiguous in K),
// B = 16 tokens of x.  Down: A = 16 tokens of h (contiguous in slots),
// B = 16 columns of 32 W_down^T rows: each lane reads CPL consecutive
// columns of each of its 8 rows and regroups them with byte permutes, so one
// set of loads feeds CPL products whose columns are CPL apart.
#include "ffn_body.hpp"
#include "launch.hpp"

namespace sfnn {

struct MfmaUpArgs {
  const f16 *w_up, *w_gate;    // [f][d]
  const f16 *b_up, *b_gate;    // [f] or null
  const f16* x;                // [B][d]
  const int32_t* ids;          // compacted ids, or null: slot s is neuron s
  const int32_t* count;        // |U|, or null: f
  const uint64_t* union_mask;  // or: the union's mask words, compacted here (ids / count unused)
  int32_t* ids_out;            // with union_mask: the union's ids (each workgroup its slots) or null
  int32_t* count_out;          // with union_mask: |U| (workgroup 0), read by k_down_mfma
  const uint64_t* mask;        // per-token gate [B][f/64] or null
  float* h;                    // [32][f] this pass's h, token-major, slot-contiguous
  float* hmax;                 // [f / 32][32] largest |h| of each 32-slot step and token
  int32_t* sid;                // [f] the row each slot reads (dropped slots: the last listed row)
  int d, f, tok0, nt;          // tokens tok0 .. tok0 + nt - 1, nt <= 16 * NB
};

struct MfmaDownArgs {
  const f16* w_down_t;         // [f][d]
  const int32_t* sid;          // as written by k_up_mfma
  const int32_t* count;
  const float* h;              // as written by k_up_mfma ([32][f])
  const float* hmax;           // as written by k_up_mfma, or null: h within fp16's range, not scaled
  float* partial;              // [KG][B][d]
  int d, f, B, tok0, nt, KG;
};

constexpr int kUpSlots = 32;
constexpr int kUpBatch = 4;  // column pairs of loads in flight per wavefront

// |U| as the sparse FFN takes it: clamped to [0, f]; null: every neuron.
__device__ __forceinline__ int slot_count(const int32_t* count, int f) {
  if (!count) return f;
  const int c = *count;
  return c < 0 ? 0 : (c > f ? f : c);
}

// One 64-column pair of this wavefront's rows and tokens: 2 K blocks.
template <int NM, int NB>
struct UpFrag {
  u32x4 w[NM][2][2];  // [matrix][tile][K block]
  u32x4 x[NB][2];     // [token tile][K block]
};

template <int NM, int NB>
__device__ __forceinline__ void up_issue(UpFrag<NM, NB>& F, const f16* (&wr)[NM][2], const f16* (&xr)[NB],
                                         int pair) {
  const int k = pair * 64;
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int s = 0; s < 2; ++s) F.w[m][t][s] = ld16_stream(wr[m][t] + k + 32 * s);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int s = 0; s < 2; ++s) F.x[nb][s] = ld16(xr[nb] + k + 32 * s);
}

template <int NM, int NB>
__device__ __forceinline__ void up_mul(const UpFrag<NM, NB>& F, const bool (&xok)[NB], f32x4 (&acc)[NM][2][NB]) {
  const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const u32x4 xv = xok[nb] ? F.x[nb][s] : z;  // tokens past the pass add nothing
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int t = 0; t < 2; ++t) acc[m][t][nb] = mfma_16x16x32(F.w[m][t][s], xv, acc[m][t][nb]);
    }
}

template <int ACT, int NB>
__global__ __launch_bounds__(512) void k_up_mfma(MfmaUpArgs a) {
  constexpr int NM = ACT == ACT_REGLU ? 2 : 1;
  __shared__ f32x4 red[8][2][NB][kWave];  // one matrix's blocks at a time
  __shared__ int s_id[kUpSlots];
  __shared__ int s_ul[kUpSlots], s_wt[8];  // the union's slots of this workgroup, scan totals
  __shared__ uint32_t s_hm[32];  // largest |h| per token (fp32 bits: non-negative floats order as integers)
  const int s0 = blockIdx.x * kUpSlots;
  int cnt;
  if (a.union_mask) {  // uniform over the launch
    cnt = union_window<kUpSlots>(a.union_mask, a.f >> 6, s0, s_ul, s_wt);
    if (blockIdx.x == 0 && threadIdx.x == 0) *a.count_out = cnt;
  } else {
    cnt = slot_count(a.count, a.f);
  }
  if (s0 >= cnt) return;  // the whole workgroup
  if (threadIdx.x < 32) s_hm[threadIdx.x] = 0u;  // ordered before the maxima by the sums' barriers
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int r = lane & 15, g = lane >> 4;
  const int d = a.d;
  // Slots past |U| and ids outside [0, f) are dropped (h = 0); they re-read
  // the last listed row, so no row outside the list is touched.
  // (compacted here: the workgroup's first slot, a listed row)
  int pad = 0;
  if (a.union_mask) {
    pad = s_ul[0];
  } else if (a.ids) {
    const int v = a.ids[cnt - 1];
    pad = v >= 0 && v < a.f ? v : 0;
  }
  const f16* wr[NM][2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int s = s0 + t * 16 + r;
    int id = a.union_mask ? s_ul[t * 16 + r] : (s < cnt ? (a.ids ? a.ids[s] : s) : -1);
    if (id >= a.f) id = -1;
    const int idc = id < 0 ? pad : id;
    if (wave == 0 && g == 0) {
      s_id[t * 16 + r] = id;
      a.sid[s] = idc;
      if (a.union_mask && a.ids_out && s < cnt) a.ids_out[s] = id;
    }
    wr[0][t] = a.w_up + (size_t)idc * d + 8 * g;
    if constexpr (NM == 2) wr[1][t] = a.w_gate + (size_t)idc * d + 8 * g;
  }
  const f16* xr[NB];
  bool xok[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int tk = nb * 16 + r;
    xok[nb] = tk < a.nt;
    xr[nb] = a.x + (size_t)(a.tok0 + (xok[nb] ? tk : 0)) * d + 8 * g;
  }
  f32x4 acc[NM][2][NB];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[m][t][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // pairs wave, wave + 8, ... in batches of kUpBatch: every batch's loads go
  // out before any of its products (a pair past the last re-reads the last)
  const int npair = d >> 6;
  const int iters = wave < npair ? (npair - wave + 7) >> 3 : 0;
  for (int b0 = 0; b0 < iters; b0 += kUpBatch) {
    UpFrag<NM, NB> F[kUpBatch];
#pragma unroll
    for (int j = 0; j < kUpBatch; ++j) up_issue(F[j], wr, xr, wave + 8 * (b0 + j < iters ? b0 + j : iters - 1));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < kUpBatch; ++j)
      if (b0 + j < iters) up_mul(F[j], xok, acc);
  }

  // the 8 wavefronts' blocks added in wavefront order; thread e-slots
  // e = threadIdx.x + 512 k, k < NB, cover 32 slots x 16 NB tokens
  constexpr int E = 2 * NB * kWave * 4;
  const float* rf = reinterpret_cast<const float*>(&red[0][0][0][0]);
  float su[NB], sg[NB];
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    if (m) __syncthreads();
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) red[wave][t][nb][lane] = acc[m][t][nb];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int e = threadIdx.x + 512 * k;
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < 8; ++w) v += rf[w * E + e];
      if (m == 0) su[k] = v; else sg[k] = v;
    }
  }
  const int words = a.f >> 6;
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    const int e = threadIdx.x + 512 * k;
    const int q = e & 3, ln = (e >> 2) & (kWave - 1), nb = (e >> 8) % NB, t = e / (256 * NB);
    const int row = t * 16 + 4 * (ln >> 4) + q;
    const int tk = nb * 16 + (ln & 15);  // tokens past the pass get h = 0 (k_down_mfma reads them)
    const int id = tk < a.nt ? s_id[row] : -1;
    float hv = 0.0f;
    if (id >= 0) {
      const float up = su[k] + (a.b_up ? (float)a.b_up[id] : 0.0f);
      if constexpr (ACT == ACT_RELU) {
        hv = up > 0.0f ? up : 0.0f;
      } else {
        const float gt = sg[k] + (a.b_gate ? (float)a.b_gate[id] : 0.0f);
        hv = (gt > 0.0f ? gt : 0.0f) * up;
      }
      if (a.mask) {
        const uint64_t wv = a.mask[(size_t)(a.tok0 + tk) * words + (id >> 6)];
        if (!((wv >> (id & 63)) & 1ull)) hv = 0.0f;  // select: gated-off neurons add nothing
      }
    }
    a.h[(size_t)tk * a.f + s0 + row] = hv;
    atomicMax(&s_hm[tk], __builtin_bit_cast(uint32_t, __builtin_fabsf(hv)));
  }
  __syncthreads();
  if (threadIdx.x < 32) a.hmax[(size_t)blockIdx.x * 32 + threadIdx.x] = __builtin_bit_cast(float, s_hm[threadIdx.x]);
}

// One 32-slot step of the down projection for this lane: 8 rows (its K
// block), CPL consecutive columns of each, and h of its tokens over the 8 slots.
template <int NB, int CPL>
struct DownFrag {
  uint32_t w[8][CPL / 2];
  f32x4 h[NB][2];  // [token tile][first, last four slots]
};

__device__ __forceinline__ void down_ids(const MfmaDownArgs& a, int st, int g, int (&id)[8]) {
  // sid holds every slot below |U| rounded up to 32 (d_ff is a multiple of 64)
  const int base = st * 32 + 8 * g;
  const u32x4 v0 = ld16(a.sid + base), v1 = ld16(a.sid + base + 4);
  id[0] = (int)v0.x; id[1] = (int)v0.y; id[2] = (int)v0.z; id[3] = (int)v0.w;
  id[4] = (int)v1.x; id[5] = (int)v1.y; id[6] = (int)v1.z; id[7] = (int)v1.w;
}

template <int NB, int CPL>
__device__ __forceinline__ void down_issue(DownFrag<NB, CPL>& F, const MfmaDownArgs& a, const int (&id)[8], int col0,
                                           const float* (&hr)[NB], int st) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const f16* src = a.w_down_t + (size_t)id[e] * a.d + col0;
    if constexpr (CPL == 8) {
      const u32x4 v = ld16_stream(src);
      F.w[e][0] = v.x; F.w[e][1] = v.y; F.w[e][2] = v.z; F.w[e][3] = v.w;
    } else {
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(src));
      F.w[e][0] = v.x; F.w[e][1] = v.y;
    }
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    F.h[nb][0] = *reinterpret_cast<const f32x4*>(hr[nb] + st * 32);
    F.h[nb][1] = *reinterpret_cast<const f32x4*>(hr[nb] + st * 32 + 4);
  }
}

__device__ __forceinline__ uint32_t pick16(uint32_t lo, uint32_t hi, int odd) {
  return odd ? ((hi & 0xffff0000u) | (lo >> 16)) : ((hi << 16) | (lo & 0xffffu));
}

// scin[nb]: the range scale of this lane's A token (n + 16 nb).
template <int NB, int CPL>
__device__ __forceinline__ void down_mul(const DownFrag<NB, CPL>& F, const float (&scin)[NB], f32x4 (&acc)[CPL][NB]) {
  u32x4 ah[NB], al[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) split_hi_lo(F.h[nb][0] * scin[nb], F.h[nb][1] * scin[nb], ah[nb], al[nb]);
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    // column i of this lane's CPL columns, over its 8 rows (K)
    u32x4 b;
    b.x = pick16(F.w[0][i >> 1], F.w[1][i >> 1], i & 1);
    b.y = pick16(F.w[2][i >> 1], F.w[3][i >> 1], i & 1);
    b.z = pick16(F.w[4][i >> 1], F.w[5][i >> 1], i & 1);
    b.w = pick16(F.w[6][i >> 1], F.w[7][i >> 1], i & 1);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      acc[i][nb] = mfma_16x16x32(ah[nb], b, acc[i][nb]);
      acc[i][nb] = mfma_16x16x32(al[nb], b, acc[i][nb]);
    }
  }
}

// Columns per lane: 8 (one 16-byte load per row) for one token tile, 4 for
// two, so the accumulators and row fragments fit 256 registers.
template <int NB>
constexpr int down_cpl() { return NB == 1 ? 8 : 4; }

template <int NB>
__global__ __launch_bounds__(512) void k_down_mfma(MfmaDownArgs a) {
  constexpr int CPL = down_cpl<NB>();
  constexpr int WC = 16 * CPL;  // columns per workgroup
  __shared__ f32x4 red[8][2][NB][kWave];
  __shared__ uint32_t s_hm[32];
  const int cnt = slot_count(a.count, a.f);
  const int cs = blockIdx.x / a.KG, kg = blockIdx.x % a.KG;  // slot group b % KG: one XCD's slots, see mfma_groups
  const int nsteps = (cnt + 31) >> 5;
  const int spg = (nsteps + a.KG - 1) / a.KG;
  const int st0 = kg * spg;
  const int st1 = st0 + spg < nsteps ? st0 + spg : nsteps;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int n = lane & 15, g = lane >> 4;
  const int col0 = cs * WC + CPL * n;
  const float* hr[NB];  // rows of tokens past the pass hold zeros
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) hr[nb] = a.h + (size_t)(nb * 16 + n) * a.f + 8 * g;
  // each token's largest |h| over this group's slots, and the range scales
  if (threadIdx.x < 32) s_hm[threadIdx.x] = 0u;
  __syncthreads();
  if (a.hmax) token_max_steps(a.hmax, st0, st1, s_hm);
  __syncthreads();
  float scin[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) scin[nb] = pow2f(-range_exp(__builtin_bit_cast(float, s_hm[nb * 16 + n])));
  f32x4 acc[CPL][NB];
#pragma unroll
  for (int i = 0; i < CPL; ++i)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[i][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // steps st0 + wave, + 8, ...: ids two steps ahead, rows one step ahead; every
  // request unconditional (the last ones re-read the current step)
  const int first = st0 + wave;
  const int iters = first < st1 ? (st1 - first + 7) >> 3 : 0;
  auto S = [&](int it) { return first + 8 * it; };
  if (iters > 0) {
    int idA[8], idB[8];
    DownFrag<NB, CPL> A, Bf;
    down_ids(a, first, g, idA);
    const int s1 = iters > 1 ? S(1) : first;
    down_ids(a, s1, g, idB);
    down_issue(A, a, idA, col0, hr, first);
    for (int it = 0; it < iters; it += 2) {
      const int sa = S(it);
      const int sb = it + 1 < iters ? S(it + 1) : sa;
      const int sc = it + 2 < iters ? S(it + 2) : sb;
      down_ids(a, sc, g, idA);
      down_issue(Bf, a, idB, col0, hr, sb);
      __builtin_amdgcn_sched_barrier(0);
      down_mul(A, scin, acc);
      if (it + 1 >= iters) break;
      const int sd = it + 3 < iters ? S(it + 3) : sc;
      down_ids(a, sd, g, idB);
      down_issue(A, a, idA, col0, hr, sc);
      __builtin_amdgcn_sched_barrier(0);
      down_mul(Bf, scin, acc);
    }
  }

  // add the 8 wavefronts' blocks in order, two column indices at a time;
  // every workgroup writes its rows (zeros when its group is empty)
  const float* rf = reinterpret_cast<const float*>(&red[0][0][0][0]);
  constexpr int E = 2 * NB * kWave * 4;
#pragma unroll
  for (int qt = 0; qt < CPL / 2; ++qt) {
    if (qt) __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) red[wave][i][nb][lane] = acc[qt * 2 + i][nb];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int e = threadIdx.x + 512 * k;
      float s = 0.0f;
#pragma unroll
      for (int w = 0; w < 8; ++w) s += rf[w * E + e];
      const int q = e & 3, ln = (e >> 2) & (kWave - 1), nb = (e >> 8) % NB, i = e / (256 * NB);
      const int tk = nb * 16 + 4 * (ln >> 4) + q;
      if (tk >= a.nt) continue;
      const int col = cs * WC + CPL * (ln & 15) + qt * 2 + i;
      a.partial[((size_t)kg * a.B + a.tok0 + tk) * a.d + col] =
          s * pow2f(range_exp(__builtin_bit_cast(float, s_hm[tk])));
    }
  }
}

// ---- host side ---------------------------------------------------------------

bool ffn_uses_mfma(const FfnLaunch& p) {
  const int def = p.wt == WT_I4 ? kMfmaMinBatchI4Default : kMfmaMinBatchDefault;
  const int thr = p.mfma_min_batch == 0 ? def : p.mfma_min_batch;
  return thr > 0 && p.batch >= thr && (p.wt == WT_F16 || p.wt == WT_I4) && p.hbuf != nullptr &&
         p.sidbuf != nullptr;
}

// Slot groups of the down projection.  Every column workgroup re-reads h of
// its slot group, and workgroup b runs on XCD b % 8, so the count is a
// multiple of 8 and block b takes slot group b % KG: each XCD then works on
// its own eighth (or sixteenth ...) of the slots, whose h stays in that XCD's
// L2 instead of streaming the whole h from the Infinity Cache once per column
// workgroup.  About 256 workgroups of 128 columns; one count for every pass
// of a call, as k_sum adds them.
int mfma_groups(int d, int max_groups) {
  const int cs = d / 128;
  int kg = 8 * ((32 + cs - 1) / cs);
  if (kg > max_groups) kg = max_groups;  // the partial buffer holds max_groups rows per token
  if (kg < 1) kg = 1;
  return kg;
}

template <int ACT, int NB>
static void mfma_pass(const FfnLaunch& p, const int32_t* ids, const int32_t* count, int tok0, int nt, int kg,
                      hipStream_t s, const uint64_t* union_mask) {
  MfmaUpArgs u;
  u.w_up = (const f16*)p.w_up;
  u.w_gate = (const f16*)p.w_gate;
  u.b_up = (const f16*)p.b_up;
  u.b_gate = (const f16*)p.b_gate;
  u.x = (const f16*)p.x;
  u.ids = ids;
  u.count = count;
  u.union_mask = union_mask;
  u.ids_out = p.ids_out;
  u.count_out = p.count_out;
  u.mask = p.mask;
  u.h = (float*)p.hbuf;
  u.hmax = p.hmax;
  u.sid = p.sidbuf;
  u.d = p.d;
  u.f = p.f;
  u.tok0 = tok0;
  u.nt = nt;
  hipLaunchKernelGGL((k_up_mfma<ACT, NB>), dim3(p.f / kUpSlots), dim3(512), 0, s, u);
  MfmaDownArgs dn;
  dn.w_down_t = (const f16*)p.w_down_t;
  dn.sid = p.sidbuf;
  dn.count = count;
  dn.h = (const float*)p.hbuf;
  dn.hmax = p.hmax;
  dn.partial = p.partial;
  dn.d = p.d;
  dn.f = p.f;
  dn.B = p.batch;
  dn.tok0 = tok0;
  dn.nt = nt;
  dn.KG = kg;
  hipLaunchKernelGGL((k_down_mfma<NB>), dim3((p.d / (16 * down_cpl<NB>())) * kg), dim3(512), 0, s, dn);
}

void launch_rows_mfma(const void* w_t, const int32_t* sid, const int32_t* count, const void* h, float* partial, int d,
                      int f, int B, int tok0, int nt, int kg, hipStream_t s) {
  MfmaDownArgs dn;
  dn.w_down_t = (const f16*)w_t;
  dn.sid = sid;
  dn.count = count;
  dn.h = (const float*)h;
  dn.hmax = nullptr;  // fp16 inputs: within range
  dn.partial = partial;
  dn.d = d;
  dn.f = f;
  dn.B = B;
  dn.tok0 = tok0;
  dn.nt = nt;
  dn.KG = kg;
  if (nt > 16)
    hipLaunchKernelGGL((k_down_mfma<2>), dim3((d / (16 * down_cpl<2>())) * kg), dim3(512), 0, s, dn);
  else
    hipLaunchKernelGGL((k_down_mfma<1>), dim3((d / (16 * down_cpl<1>())) * kg), dim3(512), 0, s, dn);
}

template <int ACT>
static void mfma_all(const FfnLaunch& p, const int32_t* ids, const int32_t* count, hipStream_t s,
                     const uint64_t* union_mask) {
  const int kg = mfma_groups(p.d, kMfmaPartRows);
  for (int tok0 = 0; tok0 < p.batch; tok0 += 32) {
    const int nt = p.batch - tok0 < 32 ? p.batch - tok0 : 32;
    if (nt > 16)
      mfma_pass<ACT, 2>(p, ids, count, tok0, nt, kg, s, union_mask);
    else
      mfma_pass<ACT, 1>(p, ids, count, tok0, nt, kg, s, union_mask);
  }
}

hipError_t launch_ffn_mfma(const FfnLaunch& p, hipStream_t s) {
  const int32_t* ids = nullptr;
  const int32_t* count = nullptr;
  if (p.wt == WT_I4) {
    const int kg = mfma_groups(p.d, kMfmaPartRows);
    if ((p.f / 32 + kg - 1) / kg * 32 > kMfmaI4MaxGroupSlots) return hipErrorInvalidValue;  // not for d_ff <= 65536
  }
  const uint64_t* um = nullptr;
  if (p.src == SRC_UNION && p.count_out) {
    // the union compacted inside the up kernel (each workgroup its slots):
    // ids_out / count_out, which the down kernel then reads
    um = p.union_mask;
    count = p.count_out;
  } else if (p.src == SRC_UNION) {
    // no place for |U| given: the compaction launch into the workspace
    return hipErrorInvalidValue;
  } else if (p.src == SRC_IDS) {
    ids = p.ids;
    count = p.count;
  }
  if (p.wt == WT_I4)
    mfma_all_i4(p, ids, count, mfma_groups(p.d, kMfmaPartRows), s, um);
  else if (p.act == ACT_RELU)
    mfma_all<ACT_RELU>(p, ids, count, s, um);
  else
    mfma_all<ACT_REGLU>(p, ids, count, s, um);
  if (p.y || p.r_out) return launch_sum(p, mfma_groups(p.d, kMfmaPartRows), s);
  return hipGetLastError();
}

}  // namespace sfnn
