// Larger batches of the gathered FFN on the matrix cores, INT4-g128 weights
// (weight-only quantisation dequantised inside the kernel, [ciyun] 2.2 量化;
// INT4 support of PowerInfer, [news]).
//
// Each 128-element group of a weight row holds signed nibbles q with one fp16
// scale s; w = q s.  The nibbles enter the matrix cores exactly (as fp16
// integers), and the scale is applied in fp32, so no weight is rounded:
//
//  k_up_mfma_i4   workgroup = 16 RT gathered rows (RT row tiles) x the
//                 pass's tokens; its 8 wavefronts split d_model into the
//                 128-wide scale groups (group w, w + 8, ...).  Per group and
//                 16x16 block: four v_mfma_f32_16x16x32_f16 on the group's
//                 nibbles (lane l takes the 32 nibbles 32 (l / 16) .. + 31 of
//                 row l % 16, one 16-byte load) and the token values, then
//                 acc += s_row * (that sum), with the
//                 workgroup's scales staged in LDS.  Blocks added in wavefront
//                 order; bias, activation and per-token select give h [token]
//                 [slot] in fp32, and the largest |h| of each token over
//                 each 32-slot step.
//  k_down_mfma_i4 workgroup = one 128-column scale group x one group of
//                 slots.  In that column group row k has a single scale s_k,
//                 so y = sum_k h_k s_k q_k: each step of 32 slots scales h by
//                 its rows' scales and by the token's power-of-two range
//                 scale (fp32; chosen from the token's largest |h| over the
//                 group's slots times the group's largest |s_k|), splits the
//                 product into two fp16 planes (22 bits, no overflow), and
//                 multiplies them with the nibbles of 8 consecutive columns
//                 per lane (4 bytes per row), regrouped per column with byte
//                 permutes.  The group's row ids and this column group's
//                 scales (at most 8192 slots) are staged in LDS, so a
//                 wavefront issues the row loads of several steps back to
//                 back.  One fp32 partial row per slot group and token,
//                 scaled back and added in a fixed order by k_sum.
//
// Workgroups of neighbouring column groups read the two 64-byte halves of the
// same 128-byte lines; with the slot group as the fast block index they run
// on one XCD (blocks b and b + KG), so a line's second half meets it in that
// L2.
#include "ffn_body.hpp"
#include "launch.hpp"

namespace sfnn {

struct MfmaUpI4Args {
  const uint8_t *q_up, *q_gate;  // [f][d/2] nibbles
  const f16 *s_up, *s_gate;      // [f][d/128] scales
  const f16 *b_up, *b_gate;      // [f] or null
  const f16* x;                  // [B][d]
  const int32_t* ids;            // compacted ids, or null: slot s is neuron s
  const int32_t* count;          // |U|, or null: f
  const uint64_t* union_mask;    // or: the union's mask words, compacted here (ids / count unused)
  int32_t* ids_out;              // with union_mask: the union's ids (each workgroup its slots) or null
  int32_t* count_out;            // with union_mask: |U| (workgroup 0), read by k_down_mfma_i4
  const uint64_t* mask;          // per-token gate [B][f/64] or null
  float* h;                      // [32][f] this pass's h, token-major, slot-contiguous
  float* hmax;                   // [f / 32][32] largest |h| of each 32-slot step and token
  int32_t* sid;                  // [f] the row each slot reads (dropped slots: the last listed row)
  int d, f, tok0, nt;
};

struct MfmaDownI4Args {
  const uint8_t* q_down_t;  // [f][d/2]
  const f16* s_down_t;      // [f][d/128]
  const int32_t* sid;
  const int32_t* count;
  const float* h;           // [32][f]
  const float* hmax;        // [f / 32][32]
  float* partial;           // [KG][B][d]
  int d, f, B, tok0, nt, KG;
};

__device__ __forceinline__ int slot_count_i4(const int32_t* count, int f) {
  if (!count) return f;
  const int c = *count;
  return c < 0 ? 0 : (c > f ? f : c);
}

// The 8 nibbles of a dword (element j in bits 4j .. 4j + 3, two's
// complement) as fp16 integers in element order, two per dword: (t ^ 8) is t
// + 8 in offset binary, fp16 0x6400 | n is 1024 + n, and 1032 is taken off.
__device__ __forceinline__ u32x4 nib8(uint32_t u) {
  const uint32_t v = u ^ 0x88888888u;
  const f16x2 bias = {(f16)1032.0f, (f16)1032.0f};
  uint32_t p[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t lo = (v >> (8 * k)) & 0xFu, hi = (v >> (8 * k + 4)) & 0xFu;
    p[k] = __builtin_bit_cast(uint32_t, bitcast<f16x2>(lo | (hi << 16) | 0x64006400u) - bias);
  }
  return u32x4{p[0], p[1], p[2], p[3]};
}

template <int NM, int RT, int NB>
struct UpI4Frag {
  u32x4 w[NM][RT];     // one 16-byte load per row tile: 32 nibbles of the group
  u32x4 x[NB][4];      // 4 x 8 token values, natural order
};

template <int ACT, int RT, int NB>
__global__ __launch_bounds__(512) void k_up_mfma_i4(MfmaUpI4Args a) {
  constexpr int NM = ACT == ACT_REGLU ? 2 : 1;
  constexpr int ROWS = 16 * RT;
  constexpr int kMaxGroups = 128;                    // d_model <= 16384
  __shared__ f32x4 red[8][2][NB][kWave];             // two row tiles at a time
  __shared__ f16 ssc[NM][kMaxGroups][ROWS];          // scales, group-major
  __shared__ int s_id[ROWS];   // neuron of each row, -1 for a dropped slot
  __shared__ int s_idc[ROWS];  // the row actually read (dropped slots: the pad row)
  __shared__ uint32_t s_hm[RT / 2][32];  // largest |h| per step and token (fp32 bits)
  __shared__ int s_ul[ROWS], s_wt[8];    // the union's slots of this workgroup, scan totals
  const int s0 = blockIdx.x * ROWS;
  int cnt;
  if (a.union_mask) {  // uniform over the launch
    cnt = union_window<ROWS>(a.union_mask, a.f >> 6, s0, s_ul, s_wt);
    if (blockIdx.x == 0 && threadIdx.x == 0) *a.count_out = cnt;
  } else {
    cnt = slot_count_i4(a.count, a.f);
  }
  if (s0 >= cnt) return;  // the whole workgroup
  if (threadIdx.x < RT / 2 * 32) s_hm[threadIdx.x / 32][threadIdx.x % 32] = 0u;  // before the first barrier
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int r = lane & 15, g = lane >> 4;
  const int d = a.d, G = d >> 7;
  // this lane's rows (one per tile); slots past |U| and ids outside [0, f)
  // are dropped (h = 0) and re-read the last listed row (compacted here: the
  // workgroup's first slot, a listed row).  All id loads go out together
  // (slots past |U| re-read the last one).
  int raw[RT + 1];
#pragma unroll
  for (int t = 0; t <= RT; ++t) {
    const int s = t < RT ? s0 + t * 16 + r : cnt - 1;
    const int sc = s < cnt ? s : cnt - 1;
    if (a.union_mask)
      raw[t] = t < RT ? s_ul[t * 16 + r] : s_ul[0];
    else
      raw[t] = a.ids ? a.ids[sc] : sc;
  }
  const int pad = raw[RT] >= 0 && raw[RT] < a.f ? raw[RT] : 0;
  const uint8_t* wr[NM][RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int s = s0 + t * 16 + r;
    int id = s < cnt ? raw[t] : -1;
    if (id >= a.f) id = -1;
    const int idc = id < 0 ? pad : id;
    if (wave == 0 && g == 0) {
      s_id[t * 16 + r] = id;
      s_idc[t * 16 + r] = idc;
      if (s < a.f) a.sid[s] = idc;  // the last workgroup's rows may run past d_ff
      if (a.union_mask && a.ids_out && s < cnt) a.ids_out[s] = id;
    }
    wr[0][t] = a.q_up + (size_t)idc * (d >> 1) + 16 * g;
    if constexpr (NM == 2) wr[1][t] = a.q_gate + (size_t)idc * (d >> 1) + 16 * g;
  }
  const f16* xr[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int tk = nb * 16 + r;
    xr[nb] = a.x + (size_t)(a.tok0 + (tk < a.nt ? tk : 0)) * d + 32 * g;
  }
  auto issue = [&](UpI4Frag<NM, RT, NB>& F, int grp) {
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int t = 0; t < RT; ++t) F.w[m][t] = ld16_stream(wr[m][t] + grp * 64);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int s = 0; s < 4; ++s) F.x[nb][s] = ld16(xr[nb] + grp * 128 + 8 * s);
  };

  // the first groups' loads go out before the scales are staged
  const int iters = wave < G ? (G - wave + 7) >> 3 : 0;
  UpI4Frag<NM, RT, NB> A, Bf;
  if (iters > 0) issue(A, wave);
  __syncthreads();  // s_idc
  {
    // every scale load goes out before the first LDS store (one round trip):
    // NM * ROWS * G <= 8192 values, at most 16 per thread; indices past the
    // end re-read the last value
    constexpr int kPer = NM * ROWS * kMaxGroups / 512;
    const int n = NM * ROWS * G;
    f16 sv[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i0 = threadIdx.x + 512 * j;
      const int i = i0 < n ? i0 : n - 1;
      const int m = i / (ROWS * G), rem = i - m * ROWS * G;
      const int row = rem / G, grp = rem - row * G;
      const f16* sp = m == 0 ? a.s_up : a.s_gate;
      sv[j] = sp[(size_t)s_idc[row] * G + grp];
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = threadIdx.x + 512 * j;
      if (i < n) {
        const int m = i / (ROWS * G), rem = i - m * ROWS * G;
        const int row = rem / G, grp = rem - row * G;
        ssc[m][grp][row] = sv[j];
      }
    }
  }
  __syncthreads();

  f32x4 acc[NM][RT][NB];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[m][t][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // tokens past the pass multiply token 0's values; their h is set to zero
  auto mul = [&](const UpI4Frag<NM, RT, NB>& F, int grp) {
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const u32x4 q = F.w[m][t];
        const u32x4 qa[4] = {nib8(q.x), nib8(q.y), nib8(q.z), nib8(q.w)};
        // scales of this lane's D rows 4g .. 4g + 3 of tile t
        const f16* sc = &ssc[m][grp][t * 16 + 4 * g];
        const f32x4 sv = {(float)sc[0], (float)sc[1], (float)sc[2], (float)sc[3]};
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < 4; ++s) p = mfma_16x16x32(qa[s], F.x[nb][s], p);
          acc[m][t][nb].x = __builtin_fmaf(sv.x, p.x, acc[m][t][nb].x);
          acc[m][t][nb].y = __builtin_fmaf(sv.y, p.y, acc[m][t][nb].y);
          acc[m][t][nb].z = __builtin_fmaf(sv.z, p.z, acc[m][t][nb].z);
          acc[m][t][nb].w = __builtin_fmaf(sv.w, p.w, acc[m][t][nb].w);
        }
      }
  };

  // groups wave, wave + 8, ...; two fragment sets in flight; every request is
  // unconditional (the last one re-reads the current group)
  if (iters > 0) {
    for (int it = 0; it < iters; it += 2) {
      const int ga = wave + 8 * it;
      const int gb = it + 1 < iters ? ga + 8 : ga;
      issue(Bf, gb);
      __builtin_amdgcn_sched_barrier(0);
      mul(A, ga);
      if (it + 1 >= iters) break;
      issue(A, it + 2 < iters ? gb + 8 : gb);
      __builtin_amdgcn_sched_barrier(0);
      mul(Bf, gb);
    }
  }

  // the 8 wavefronts' blocks added in wavefront order, two tiles at a time;
  // thread e-slots e = threadIdx.x + 512 k (k < NB) cover 2 tiles x 16 NB tokens
  constexpr int E = 2 * NB * kWave * 4;
  const float* rf = reinterpret_cast<const float*>(&red[0][0][0][0]);
  const int words = a.f >> 6;
#pragma unroll
  for (int tp = 0; tp < RT / 2; ++tp) {
    float su[NB], sg[NB];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) red[wave][i][nb][lane] = acc[m][2 * tp + i][nb];
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
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int e = threadIdx.x + 512 * k;
      const int q = e & 3, ln = (e >> 2) & (kWave - 1), nb = (e >> 8) % NB, i = e / (256 * NB);
      const int row = (2 * tp + i) * 16 + 4 * (ln >> 4) + q;
      const int tk = nb * 16 + (ln & 15);  // tokens past the pass get h = 0 (k_down_mfma_i4 reads them)
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
      if (s0 + row < a.f) a.h[(size_t)tk * a.f + s0 + row] = hv;
      atomicMax(&s_hm[tp][tk], __builtin_bit_cast(uint32_t, __builtin_fabsf(hv)));
    }
  }
  __syncthreads();
  if (threadIdx.x < RT / 2 * 32) {
    const int st = s0 / 32 + threadIdx.x / 32;  // the last workgroup's steps may run past d_ff
    if (st < a.f / 32) a.hmax[(size_t)st * 32 + threadIdx.x % 32] = __builtin_bit_cast(float, s_hm[threadIdx.x / 32][threadIdx.x % 32]);
  }
}

// Slots staged in LDS by a down workgroup: their row ids and this column
// group's scales (48 KB).  One slot group never holds more: d_ff <= 65536 is
// at most 2048 steps of 32 slots, and there are at least 8 slot groups
// (mfma_groups), so a group has at most 256 steps.
constexpr int kDownChunk = kMfmaI4MaxGroupSlots;

// Steps of loads a wavefront issues before multiplying (registers allow four
// with one token tile, three with two).
template <int NB>
constexpr int down_i4_batch() { return NB == 1 ? 4 : 3; }

// One 32-slot step of the down projection for this lane: its 8 rows (K
// block), 8 consecutive columns of each (one dword of nibbles), and h of its
// tokens over the 8 slots.
template <int NB>
struct DownI4Frag {
  uint32_t w[8];
  f32x4 h[NB][2];
};

// Loads of step st; lid holds the chunk's row ids (slot c0 * 32 onwards).
template <int NB>
__device__ __forceinline__ void down_issue_i4(DownI4Frag<NB>& F, const MfmaDownI4Args& a, const int* lid, int c0,
                                              int boff, const float* (&hr)[NB], int st, int g) {
  const int* ip = lid + (st - c0) * 32 + 8 * g;
  const int4 i0 = *reinterpret_cast<const int4*>(ip);
  const int4 i1 = *reinterpret_cast<const int4*>(ip + 4);
  const int id[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
#pragma unroll
  for (int e = 0; e < 8; ++e)
    F.w[e] = *reinterpret_cast<const uint32_t*>(a.q_down_t + (size_t)id[e] * (a.d >> 1) + boff);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    F.h[nb][0] = *reinterpret_cast<const f32x4*>(hr[nb] + st * 32);
    F.h[nb][1] = *reinterpret_cast<const f32x4*>(hr[nb] + st * 32 + 4);
  }
}

// sc: the 8 rows' scales of this column group (LDS); scin[nb]: the range
// scale of this lane's A token (n + 16 nb).
template <int NB>
__device__ __forceinline__ void down_mul_i4(const DownI4Frag<NB>& F, const f16* sc, const float (&scin)[NB],
                                            f32x4 (&acc)[8][NB]) {
  const u32x4 sraw = *reinterpret_cast<const u32x4*>(sc);
  const f16x2 s01 = bitcast<f16x2>(sraw.x), s23 = bitcast<f16x2>(sraw.y);
  const f16x2 s45 = bitcast<f16x2>(sraw.z), s67 = bitcast<f16x2>(sraw.w);
  // A operands: h of each token tile times its rows' scales, as two fp16 planes
  u32x4 ah[NB], al[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const f32x4 h0 = F.h[nb][0] * scin[nb], h1 = F.h[nb][1] * scin[nb];
    const f32x4 p0 = {h0.x * (float)s01.x, h0.y * (float)s01.y, h0.z * (float)s23.x, h0.w * (float)s23.y};
    const f32x4 p1 = {h1.x * (float)s45.x, h1.y * (float)s45.y, h1.z * (float)s67.x, h1.w * (float)s67.y};
    split_hi_lo(p0, p1, ah[nb], al[nb]);
  }
  // B operands: column i over the 8 rows, nibbles as fp16 integers.  Offset
  // binary first (t ^ 8 = t + 8); a row pair's byte k sits in the low bytes of
  // each half of perm's result, its low nibble is column 2k, its high one 2k+1.
  uint32_t v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = F.w[e] ^ 0x88888888u;
  const f16x2 bias = {(f16)1032.0f, (f16)1032.0f};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t lo[4], hi[4];
#pragma unroll
    for (int rp = 0; rp < 4; ++rp) {
      const uint32_t sel = 0x0c000c00u | (uint32_t)k | ((uint32_t)(4 + k) << 16);
      const uint32_t t = __builtin_amdgcn_perm(v[2 * rp + 1], v[2 * rp], sel);
      const f16x2 ql = bitcast<f16x2>((t & 0x000F000Fu) | 0x64006400u) - bias;
      const f16x2 qh = bitcast<f16x2>(((t >> 4) & 0x000F000Fu) | 0x64006400u) - bias;
      lo[rp] = __builtin_bit_cast(uint32_t, ql);
      hi[rp] = __builtin_bit_cast(uint32_t, qh);
    }
    const u32x4 b0 = {lo[0], lo[1], lo[2], lo[3]};
    const u32x4 b1 = {hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      acc[2 * k][nb] = mfma_16x16x32(ah[nb], b0, acc[2 * k][nb]);
      acc[2 * k][nb] = mfma_16x16x32(al[nb], b0, acc[2 * k][nb]);
      acc[2 * k + 1][nb] = mfma_16x16x32(ah[nb], b1, acc[2 * k + 1][nb]);
      acc[2 * k + 1][nb] = mfma_16x16x32(al[nb], b1, acc[2 * k + 1][nb]);
    }
  }
}

template <int NB>
__global__ __launch_bounds__(512) void k_down_mfma_i4(MfmaDownI4Args a) {
  __shared__ f32x4 red[8][2][NB][kWave];
  __shared__ __align__(16) int lid[kDownChunk];  // the group's row ids
  __shared__ __align__(16) f16 lsc[kDownChunk];  // their scales in this column group
  __shared__ uint32_t s_hm[32];                  // largest |h| per token over the group's steps (fp32 bits)
  __shared__ uint32_t s_sm;                      // largest |s_k| over the group's rows (fp32 bits)
  const int cnt = slot_count_i4(a.count, a.f);
  // slot group b % KG (one XCD's slots, see mfma_groups); neighbouring column
  // groups b and b + KG share an XCD and the halves of 128-byte lines
  const int cs = blockIdx.x / a.KG, kg = blockIdx.x % a.KG;
  const int nsteps = (cnt + 31) >> 5;
  const int spg = (nsteps + a.KG - 1) / a.KG;
  const int st0 = kg * spg;
  const int st1 = st0 + spg < nsteps ? st0 + spg : nsteps;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int n = lane & 15, g = lane >> 4;
  const int boff = cs * 64 + 4 * n;  // this lane's 8 columns cs*128 + 8n .. + 7, in bytes
  const float* hr[NB];  // rows of tokens past the pass hold zeros
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) hr[nb] = a.h + (size_t)(nb * 16 + n) * a.f + 8 * g;
  f32x4 acc[8][NB];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[i][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  constexpr int PER = kDownChunk / 512;
  constexpr int NBT = down_i4_batch<NB>();
  const int G = a.d >> 7;
  if (threadIdx.x < 32) s_hm[threadIdx.x] = 0u;
  if (threadIdx.x == 0) s_sm = 0u;
  __syncthreads();
  float scin[NB] = {};
  if (st0 < st1) {  // workgroup-uniform; st1 - st0 <= kDownChunk / 32 (the host checks)
    const int c0 = st0, c1 = st1;
    const int ns = (c1 - c0) * 32;  // slots of this group (sid holds them all)
    {
      // ids, then their scales: every load of a kind goes out before any use
      int idv[PER];
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int i = threadIdx.x + 512 * j;
        idv[j] = a.sid[c0 * 32 + (i < ns ? i : ns - 1)];
      }
      f16 sv[PER];
#pragma unroll
      for (int j = 0; j < PER; ++j) sv[j] = a.s_down_t[(size_t)idv[j] * G + cs];
      token_max_steps(a.hmax, c0, c1, s_hm);
      float sm = 0.0f;
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int i = threadIdx.x + 512 * j;
        if (i < ns) {
          lid[i] = idv[j];
          lsc[i] = sv[j];
        }
        sm = __builtin_fmaxf(sm, __builtin_fabsf((float)sv[j]));  // re-read values are the group's too
      }
      atomicMax(&s_sm, __builtin_bit_cast(uint32_t, sm));
    }
    __syncthreads();
    const float smax = __builtin_bit_cast(float, s_sm);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      scin[nb] = pow2f(-range_exp(__builtin_bit_cast(float, s_hm[nb * 16 + n]) * smax));
    // steps c0 + wave, + 8, ... in batches of NBT: every batch's loads go out
    // before any of its products (a step past the last re-reads the last)
    const int first = c0 + wave;
    const int iters = first < c1 ? (c1 - first + 7) >> 3 : 0;
    for (int b0 = 0; b0 < iters; b0 += NBT) {
      DownI4Frag<NB> F[NBT];
#pragma unroll
      for (int j = 0; j < NBT; ++j)
        down_issue_i4(F[j], a, lid, c0, boff, hr, first + 8 * (b0 + j < iters ? b0 + j : iters - 1), g);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < NBT; ++j)
        if (b0 + j < iters) down_mul_i4(F[j], lsc + (first + 8 * (b0 + j) - c0) * 32 + 8 * g, scin, acc);
    }
  }
  const float smax = __builtin_bit_cast(float, s_sm);  // 0 for an empty group: its rows are zeros

  // add the 8 wavefronts' blocks in order, two columns at a time; every
  // workgroup writes its rows (zeros when its slot group is empty)
  const float* rf = reinterpret_cast<const float*>(&red[0][0][0][0]);
  constexpr int E = 2 * NB * kWave * 4;
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) {
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
      const int col = cs * 128 + 8 * (ln & 15) + qt * 2 + i;
      a.partial[((size_t)kg * a.B + a.tok0 + tk) * a.d + col] =
          s * pow2f(range_exp(__builtin_bit_cast(float, s_hm[tk]) * smax));
    }
  }
}

// ---- host side ---------------------------------------------------------------

// Row tiles per up workgroup.  Every workgroup reads all of the pass's x, so
// the more rows it takes the less x traffic per weight byte, but the grid
// should also come out at a whole number of workgroups per CU.  ReLU: 64 rows
// with one token tile, 96 with two (OPT-175B's d_ff: 768 and 512 workgroups;
// measured 6-8% faster than 128 and 64 rows at batches 4-8 and 4% at 32);
// ReGLU (two matrices): 64 rows, half that with two token tiles (registers).
template <int ACT, int NB>
constexpr int up_rt_i4() { return ACT == ACT_REGLU ? 4 / NB : (NB == 1 ? 4 : 6); }

template <int ACT, int NB>
static void mfma_pass_i4(const FfnLaunch& p, const int32_t* ids, const int32_t* count, int tok0, int nt, int kg,
                         hipStream_t s, const uint64_t* union_mask) {
  constexpr int RT = up_rt_i4<ACT, NB>();
  MfmaUpI4Args u;
  u.q_up = (const uint8_t*)p.w_up;
  u.q_gate = (const uint8_t*)p.w_gate;
  u.s_up = (const f16*)p.s_up;
  u.s_gate = (const f16*)p.s_gate;
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
  hipLaunchKernelGGL((k_up_mfma_i4<ACT, RT, NB>), dim3((p.f + 16 * RT - 1) / (16 * RT)), dim3(512), 0, s, u);
  MfmaDownI4Args dn;
  dn.q_down_t = (const uint8_t*)p.w_down_t;
  dn.s_down_t = (const f16*)p.s_down_t;
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
  hipLaunchKernelGGL((k_down_mfma_i4<NB>), dim3((p.d / 128) * kg), dim3(512), 0, s, dn);
}

template <int ACT>
static void mfma_all_i4_act(const FfnLaunch& p, const int32_t* ids, const int32_t* count, int kg, hipStream_t s,
                            const uint64_t* union_mask) {
  for (int tok0 = 0; tok0 < p.batch; tok0 += 32) {
    const int nt = p.batch - tok0 < 32 ? p.batch - tok0 : 32;
    if (nt > 16)
      mfma_pass_i4<ACT, 2>(p, ids, count, tok0, nt, kg, s, union_mask);
    else
      mfma_pass_i4<ACT, 1>(p, ids, count, tok0, nt, kg, s, union_mask);
  }
}

void mfma_all_i4(const FfnLaunch& p, const int32_t* ids, const int32_t* count, int kg, hipStream_t s,
                 const uint64_t* union_mask) {
  if (p.act == ACT_RELU)
    mfma_all_i4_act<ACT_RELU>(p, ids, count, kg, s, union_mask);
  else
    mfma_all_i4_act<ACT_REGLU>(p, ids, count, kg, s, union_mask);
}

}  // namespace sfnn
