// Column-tiled down projection over a list of rows:
//   y[t][c] = bias[c] + sum over slots j < count of  h[t][j] * W[row_j][c]
// W is row-major [rows][d]: the FFN's neuron-major W_down^T (row i is column i
// of W_down), or an input-major projection w_t.  Only the listed rows are
// read: a zero activation zeroes the whole row it multiplies, so that row
// need not be loaded at all (53ai.com sparsity survey, section 激活稀疏).
//
// A workgroup owns one tile of TB = 16 * LPR bytes (a whole 128-byte line
// where the row allows) of the rows of one row group: the listed slots are
// cut into RG equal runs, so a launch has tiles * RG workgroups whatever the
// row length.  LPR lanes cover a row's tile (one 16-byte load each), a
// wavefront covers 64 / LPR rows per load, eight wavefronts 512 / LPR.  With
// one row group the workgroup ends holding the complete sums of its columns
// and writes y directly.  With several, each writes its group's column sums
// to a partial row, and a small launch after it (k_sum) adds the RG partial
// rows in group order (deterministic) into y and the residual row.  (Adding
// them inside the launch, by the last group of a tile to arrive, needs a
// device-scope release from every workgroup, which writes back and
// invalidates the L2 of its XCD: far slower than the extra launch.)
//
// Pipelining: slots are taken in chunks of KB rows per lane; the row ids of
// chunk c+2 and the weights of chunk c+1 are requested before chunk c is
// used, so a lane always has one or two chunks of 16-byte loads in flight and
// the id of a row arrives before its weight load is issued.
//
// Reduction: every lane adds its rows in slot order; lanes that share a column
// are then added with row rotations inside each 16-lane row, the four rows and
// eight wavefronts through LDS, always in the same order (deterministic, no
// atomics).
#pragma once
#include "common.hpp"
#include "launch.hpp"

namespace sfnn {

// Source of the coefficient of slot j for token t.
enum { CO_H = 0, CO_X16 = 1, CO_X32 = 2 };  // h[t][j] fp32 | x[t][row_j] fp16 | fp32

// A row list a workgroup builds in its own LDS (the input-sparse GEMV's
// single-launch form): the count in the first word of the dynamic LDS, the
// 16-bit row ids from byte 16 on.
__device__ __forceinline__ int* lds_list_base() {
  extern __shared__ __align__(16) int lds_dyn[];
  return lds_dyn;
}
__device__ __forceinline__ uint16_t* lds_list_ids() { return reinterpret_cast<uint16_t*>(lds_list_base() + 4); }
// The packed form (one token): entry j = row id | fp16 coefficient bits << 16.
__device__ __forceinline__ uint32_t* lds_list_packed() { return reinterpret_cast<uint32_t*>(lds_list_base() + 4); }

struct DownArgs {
  const uint8_t* w;      // [n_rows][d] storage rows (INT4: [n_rows][d/2] nibbles)
  const f16* s;          // INT4: [n_rows][d/128] fp16 scales
  const int32_t* ids;    // row of slot j (null: slot j is row j)
  const int32_t* count;  // device slot count (null: n_slots)
  int n_slots;           // slots when count is null, and the upper clamp for *count
  int n_rows;            // rows of w: listed ids outside [0, n_rows) add nothing
  const void* co;        // coefficients: h [B][co_stride] fp32, or x [B][co_stride]
  int co_stride;
  const void* bias;      // [d] (bias_f32 ? fp32 : fp16) or null
  int bias_f32;
  float* y;              // [B][d] or null
  const float* r_in;     // residual add r_out = r_in + y (null to skip)
  float* r_out;
  int d, tok0, nt;
  int rg;                // row groups (>= 1)
  float* part;           // rg > 1: partial rows [rg][batch][d] (k_sum's layout)
  int batch;             // tokens of the whole call (the partial rows' stride)
};

template <int WT>
constexpr int cols_per_vec() { return WT == WT_F32 ? 4 : (WT == WT_F16 ? 8 : 32); }

// Bytes of one row (without INT4 scales).
__host__ __device__ inline int down_row_bytes(int wt, int d) { return wt == WT_F32 ? 4 * d : (wt == WT_F16 ? 2 * d : d / 2); }

// Tile of workgroup vb < ntiles.  Workgroups are dealt to the 8 XCDs in turn
// (vb % 8); the 128 / TB tiles that share a 128-byte line of every row go to
// consecutive workgroups of one XCD.
__device__ __forceinline__ int down_tile(int vb, int ntiles, int per_line) {
  if (per_line <= 1 || ntiles % (8 * per_line)) return vb;
  const int xcd = vb & 7, k = vb >> 3;        // k-th workgroup on this XCD
  const int per_xcd = ntiles >> 3;            // tiles per XCD (a multiple of per_line)
  return xcd * per_xcd + k;
}

// Work item vb < ntiles * rg: row group vb / ntiles, tile down_tile(vb % ntiles).
__device__ __forceinline__ void down_item(int vb, int ntiles, int per_line, int& tile, int& grp) {
  grp = vb / ntiles;
  tile = down_tile(vb - grp * ntiles, ntiles, per_line);
}

constexpr int kDownThreads = 512;
#ifndef SFNN_DOWN_STREAM
#define SFNN_DOWN_STREAM 0  // 1: weight loads with the streaming hint
#endif

// Rows per lane per chunk (two chunks of 16-byte loads in flight): 8, or 4
// where the token group's accumulators leave fewer registers.
#ifndef SFNN_DOWN_KB
#define SFNN_DOWN_KB 4
#endif
template <int WT, int NT>
constexpr int down_kb() { return (NT <= 2 && NT * cols_per_vec<WT>() <= 32) ? SFNN_DOWN_KB : 4; }

// The LDS-list kernels' loop: 1, batches (loop_batches); 0, the prefetching
// loop of the other kernels.
#ifndef SFNN_DOWN_BATCHES
#define SFNN_DOWN_BATCHES 1
#endif

template <int WT, int NT, int LPR>
struct DownRed {
  static constexpr int CPL = cols_per_vec<WT>();
  static constexpr int NW = kDownThreads / kWave;
  static constexpr int floats = NW * 4 * LPR * NT * CPL;  // [wave][row16][lane c][t][col]
};

// One workgroup's work item, in phases:
//   count()   the slot count (a scalar load);
//   ids01()   the row ids of chunks 0 and 1, read without waiting for the
//             count (the id list holds n_slots entries; ids past the count
//             are read but never used);
//   first()   chunk 0's weights and coefficients;
//   loop()    every chunk: the ids two chunks ahead and the weights one chunk
//             ahead go out before the chunk is used;
//   finish()  the reduction and y / the residual row.
// LISTED: rows come from a.ids (else slot j is row j), a compile-time choice
// so the id loads are never inside a branch (a load in a branch makes every
// later wait cover all loads in flight).  LDSL: the ids and the count come
// from the workgroup's own LDS list instead (lds_list_base): 1, 16-bit ids;
// 2, packed entries that carry the one token's coefficient too, so the loop's
// only global loads are weights.  Every load is unconditional: slots past the
// count read row 0's tile and are cancelled at use, and the loop leaves by
// break.
template <int WT, int NT, int LPR, int CO, bool LISTED, int LDSL = 0>
struct DownTile {
  static_assert(LDSL != 2 || (NT == 1 && WT == WT_F16 && CO == CO_X16),
                "packed list entries carry one fp16 coefficient");
  static constexpr int CPL = cols_per_vec<WT>();
  static constexpr int NW = kDownThreads / kWave;
  static constexpr int RPW = kWave / LPR;  // rows per wavefront per step
  static constexpr int RPS = NW * RPW;     // rows per workgroup per step
  static constexpr int KB = down_kb<WT, NT>();
  static_assert(LPR == 1 || LPR == 2 || LPR == 4 || LPR == 8, "lanes per row");

  int tile, grp, rr, j0, n, nch, sgrp, ngrp;  // n: slots of this row group, from slot j0
  int craw;              // the slot count as read (used by run())
  size_t rowb, cofs;
  int idb[2][KB];       // ids of the chunks ahead
  u32x4 wv[2][KB];      // weights of the chunk in use and the next one
  float hv[2][KB][NT];  // coefficients
  float sv[2][KB];      // INT4 scales
  float acc[NT][CPL];
  float sb[WT == WT_I4 ? NT : 1];
  float ob, orv;        // with one row group: this thread's output column's bias and residual
  static_assert(NT * LPR * CPL <= kDownThreads, "one output column per thread at most");

  // What does not wait for the count: the tile, this lane's rows and column,
  // the count's own load, and (one row group) the bias and residual of the
  // output column this thread writes in finish(), so that neither load waits
  // at the end.  The run starts at slot j0 = 0 here; run() sets it for row
  // groups.  has == false: a workgroup with no tile of its own (n = 0: it
  // reads slot 0's row of tile 0 and writes nothing).
  __device__ __forceinline__ void setup(const DownArgs& a, int tile_, int grp_, bool has) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int c = lane % LPR;
    tile = has ? tile_ : 0;
    grp = has ? grp_ : 0;
    rr = wave * RPW + lane / LPR;
    const int col = (tile * LPR + c) * CPL;  // first output column of this lane
    rowb = (size_t)down_row_bytes(WT, a.d);
    cofs = (size_t)down_row_bytes(WT, col);  // byte offset of the lane's 16 bytes
    sgrp = col / 128;
    ngrp = a.d / 128;
    if constexpr (LDSL)
      craw = lds_list_base()[0];
    else
      craw = a.count ? *a.count : a.n_slots;
    j0 = 0;
    n = 0;
    nch = 0;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int k = 0; k < CPL; ++k) acc[t][k] = 0.0f;
      if constexpr (WT == WT_I4) sb[t] = 0.0f;
    }
    ob = orv = 0.0f;
    constexpr int TE = LPR * CPL;
    const int e = threadIdx.x, t = e / TE;
    if (a.rg == 1 && e < NT * TE && t < a.nt) {
      const int cidx = tile * TE + e % TE;
      if (a.bias)
        ob = a.bias_f32 ? reinterpret_cast<const float*>(a.bias)[cidx]
                        : (float)reinterpret_cast<const f16*>(a.bias)[cidx];
      if (a.r_in) orv = a.r_in[(size_t)(a.tok0 + t) * a.d + cidx];
    }
  }

  // This row group's run of slots, j0 .. j0 + n - 1, from the count.
  __device__ __forceinline__ void run(const DownArgs& a, bool has) {
    const int na = craw < 0 ? 0 : (craw > a.n_slots ? a.n_slots : craw);
    const int spr = (na + a.rg - 1) / a.rg;
    j0 = grp * spr;
    n = na - j0 < spr ? na - j0 : spr;
    if (n < 0) n = 0;
    if (!has) n = 0;
    if (j0 >= a.n_slots) j0 = a.n_slots - 1;  // an empty run past the list (its reads stay in bounds)
    nch = (n + RPS * KB - 1) / (RPS * KB);  // chunks of KB steps
  }

  // the row of an id register (packed entries: the low 16 bits)
  __device__ __forceinline__ static int row_of(int e) {
    if constexpr (LDSL == 2)
      return e & 0xffff;
    else
      return e;
  }

  // slot of the run's j-th entry, clamped into the run (an empty run: j0)
  __device__ __forceinline__ int slot_clamp(const DownArgs& a, int j) const {
    const int s = j0 + (j < n ? j : (n > 0 ? n - 1 : 0));
    return s < a.n_slots ? s : a.n_slots - 1;
  }

  // ids depend on the slot only (not on the count), so they can go out
  // before the count has arrived; past the list they re-read its last entry
  __device__ __forceinline__ void issue_ids(const DownArgs& a, int ch, int (&dst)[KB]) const {
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const int j = j0 + (ch * KB + k) * RPS + rr;
      const int jc = j < a.n_slots ? j : a.n_slots - 1;
      if constexpr (LDSL == 2)
        dst[k] = (int)lds_list_packed()[jc];
      else if constexpr (LDSL == 1)
        dst[k] = lds_list_ids()[jc];
      else if constexpr (LISTED)
        dst[k] = a.ids[jc];
      else
        dst[k] = jc;
    }
  }

  __device__ __forceinline__ void issue_w(const DownArgs& a, int ch, const int (&id)[KB], u32x4 (&w)[KB],
                                          float (&h)[KB][NT], float (&sc)[KB]) const {
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const int i = row_of(id[k]);
      const bool live = (ch * KB + k) * RPS + rr < n;
      const int ic = (live && (unsigned)i < (unsigned)a.n_rows) ? i : 0;
      // a plain (cached) load: the other tiles of this 128-byte line are
      // read by neighbouring workgroups of the same XCD, from its L2
#if SFNN_DOWN_STREAM
      w[k] = ld16_stream(a.w + (size_t)ic * rowb + cofs);
#else
      w[k] = ld16(a.w + (size_t)ic * rowb + cofs);
#endif
      if constexpr (WT == WT_I4) sc[k] = (float)a.s[(size_t)ic * ngrp + sgrp];
      const int jc = slot_clamp(a, (ch * KB + k) * RPS + rr);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int tc = t < a.nt ? a.tok0 + t : a.tok0;
        if constexpr (LDSL == 2) {
          h[k][t] = (float)__builtin_bit_cast(f16, (uint16_t)((uint32_t)id[k] >> 16));
          continue;  // the coefficient came with the id
        }
        if constexpr (CO == CO_H) {
          h[k][t] = reinterpret_cast<const float*>(a.co)[(size_t)tc * a.co_stride + jc];
        } else if constexpr (CO == CO_X16) {
          h[k][t] = (float)reinterpret_cast<const f16*>(a.co)[(size_t)tc * a.co_stride + ic];
        } else {
          h[k][t] = reinterpret_cast<const float*>(a.co)[(size_t)tc * a.co_stride + ic];
        }
      }
    }
  }

  __device__ __forceinline__ void use(const DownArgs& a, int ch, const int (&id)[KB], const u32x4 (&w)[KB],
                                      const float (&h)[KB][NT], const float (&sc)[KB]) {
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const int j = (ch * KB + k) * RPS + rr;
      const bool ok = j < n && (unsigned)row_of(id[k]) < (unsigned)a.n_rows;
      float hk[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) hk[t] = (ok && t < a.nt) ? h[k][t] : 0.0f;  // a select: nothing else enters
      if constexpr (WT == WT_I4) {
        // nibbles in offset binary (n = t + 8) enter as fp16 subnormals with
        // no conversion: masked in place in bits 0-3 of a half a nibble is the
        // value n 2^-24, in bits 4-7 it is 16 n 2^-24 (see vec_i4), and the
        // fp16 operand of a mixed fma is exact in fp32; the coefficient
        // carries 2^24 or 2^20 to match.  The 8 sum(h s) the offset adds to
        // every column comes off in finish().
        float hs[NT], h24[NT], h20[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          hs[t] = ok ? hk[t] * sc[k] : 0.0f;
          sb[t] += hs[t];
          h24[t] = hs[t] * 16777216.0f;
          h20[t] = hs[t] * 1048576.0f;
        }
        const uint32_t q[4] = {w[k].x, w[k].y, w[k].z, w[k].w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const uint32_t v = q[m] ^ 0x88888888u, sh = v >> 8;
          const f16x2 p04 = bitcast<f16x2>(v & 0x000F000Fu);   // columns 8m, 8m+4
          const f16x2 p15 = bitcast<f16x2>(v & 0x00F000F0u);   // 8m+1, 8m+5 (x16)
          const f16x2 p26 = bitcast<f16x2>(sh & 0x000F000Fu);  // 8m+2, 8m+6
          const f16x2 p37 = bitcast<f16x2>(sh & 0x00F000F0u);  // 8m+3, 8m+7 (x16)
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            float* c = &acc[t][8 * m];
            c[0] = __builtin_fmaf(h24[t], (float)p04.x, c[0]);
            c[4] = __builtin_fmaf(h24[t], (float)p04.y, c[4]);
            c[1] = __builtin_fmaf(h20[t], (float)p15.x, c[1]);
            c[5] = __builtin_fmaf(h20[t], (float)p15.y, c[5]);
            c[2] = __builtin_fmaf(h24[t], (float)p26.x, c[2]);
            c[6] = __builtin_fmaf(h24[t], (float)p26.y, c[6]);
            c[3] = __builtin_fmaf(h20[t], (float)p37.x, c[3]);
            c[7] = __builtin_fmaf(h20[t], (float)p37.y, c[7]);
          }
        }
      } else {
        const u32x4 wz = ok ? w[k] : u32x4{0u, 0u, 0u, 0u};
        float e[CPL];
        if constexpr (WT == WT_F32) {
          e[0] = bitcast<float>(wz.x);
          e[1] = bitcast<float>(wz.y);
          e[2] = bitcast<float>(wz.z);
          e[3] = bitcast<float>(wz.w);
        } else {
          const uint32_t u[4] = {wz.x, wz.y, wz.z, wz.w};
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const f16x2 hh = bitcast<f16x2>(u[m]);
            e[2 * m] = (float)hh.x;
            e[2 * m + 1] = (float)hh.y;
          }
        }
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int b = 0; b < CPL; ++b) acc[t][b] = __builtin_fmaf(hk[t], e[b], acc[t][b]);
      }
    }
  }

  __device__ __forceinline__ void ids01(const DownArgs& a) {
    issue_ids(a, 0, idb[0]);
    issue_ids(a, 1, idb[1]);
  }

  __device__ __forceinline__ void first(const DownArgs& a) { issue_w(a, 0, idb[0], wv[0], hv[0], sv[0]); }

  // one chunk: idc holds chunk cc's ids (replaced by chunk cc+2's), idn chunk
  // cc+1's
  __device__ __forceinline__ void step(const DownArgs& a, int cc, int (&idc)[KB], const int (&idn)[KB],
                                       const u32x4 (&wc)[KB], const float (&hc)[KB][NT], const float (&sc)[KB],
                                       u32x4 (&wn)[KB], float (&hn)[KB][NT], float (&sn)[KB]) {
    int cur[KB];
#pragma unroll
    for (int k = 0; k < KB; ++k) cur[k] = idc[k];
    issue_ids(a, cc + 2, idc);
    issue_w(a, cc + 1, idn, wn, hn, sn);
    __builtin_amdgcn_sched_barrier(0);  // the next requests go out before this chunk is used
    use(a, cc, cur, wc, hc, sc);
  }

  // every chunk (at least one: with n = 0 it adds nothing)
  __device__ __forceinline__ void loop(const DownArgs& a) {
    for (int ch = 0;; ch += 2) {
      step(a, ch, idb[0], idb[1], wv[0], hv[0], sv[0], wv[1], hv[1], sv[1]);
      if (ch + 1 >= nch) break;
      step(a, ch + 1, idb[1], idb[0], wv[1], hv[1], sv[1], wv[0], hv[0], sv[0]);
      if (ch + 2 >= nch) break;
    }
  }

  // The LDS-list form: batches of KB rows per lane, ids (from LDS),
  // weights and coefficients requested together and used at once; no
  // requests carried from one batch to the next (a carried buffer makes the
  // compiler drain every load at the loop head anyway).
  __device__ __forceinline__ void loop_batches(const DownArgs& a) {
    for (int ch = 0; ch < nch; ++ch) {
      int id[KB];
      u32x4 w[KB];
      float h[KB][NT];
      float sc[KB];
      issue_ids(a, ch, id);
      issue_w(a, ch, id, w, h, sc);
      use(a, ch, id, w, h, sc);
    }
  }

  // red: DownRed<WT, NT, LPR>::floats of LDS.  Every thread of the workgroup
  // calls it (one barrier); has == false writes nothing.
  __device__ __forceinline__ void finish(const DownArgs& a, float* red, bool has) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    if constexpr (WT == WT_I4) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int k = 0; k < CPL; ++k) acc[t][k] = __builtin_fmaf(-8.0f, sb[t], acc[t][k]);
    }
    // lanes of one 16-lane row that share a column chunk (lane % LPR): rotate-add
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int k = 0; k < CPL; ++k) {
        float v = acc[t][k];
        v += dpp_f<0x128>(v);                          // row_ror:8
        if constexpr (LPR <= 4) v += dpp_f<0x124>(v);  // row_ror:4
        if constexpr (LPR <= 2) v += dpp_f<0x122>(v);  // row_ror:2
        if constexpr (LPR == 1) v += dpp_f<0x121>(v);  // row_ror:1
        acc[t][k] = v;
      }
    // red[wave][row16][c][t][k]: lanes 16 r + c (c < LPR) hold the row sums
    const int r16 = lane >> 4, l16 = lane & 15;
    if (l16 < LPR) {
      float* dst = red + ((((size_t)wave * 4 + r16) * LPR + l16) * NT) * CPL;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int k = 0; k < CPL; k += 4)
          *reinterpret_cast<f32x4*>(dst + t * CPL + k) =
              f32x4{acc[t][k], acc[t][k + 1], acc[t][k + 2], acc[t][k + 3]};
    }
    __syncthreads();
    constexpr int TE = LPR * CPL;  // columns of the tile
    if (!has) return;
    const bool whole = a.rg == 1;  // workgroup-uniform
    for (int e = threadIdx.x; e < NT * TE; e += kDownThreads) {
      const int t = e / TE, ce = e % TE;
      const int cl = ce / CPL, k = ce % CPL;
      float s = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int r = 0; r < 4; ++r) s += red[((((size_t)w * 4 + r) * LPR + cl) * NT + t) * CPL + k];
      if (t < a.nt) {
        const int cidx = tile * TE + ce;
        if (whole) {
          // y / the residual row from the bias and residual read in setup()
          const float v = ob + s;
          const size_t o = (size_t)(a.tok0 + t) * a.d + cidx;
          if (a.y) a.y[o] = v;
          if (a.r_in) a.r_out[o] = orv + v;
        } else {
          a.part[((size_t)grp * a.batch + a.tok0 + t) * a.d + cidx] = s;
        }
      }
    }
  }
};

// One work item on its own (k_down; with LDSL, after the workgroup built its
// row list).
template <int WT, int NT, int LPR, int CO, bool LISTED, int LDSL = 0>
__device__ __forceinline__ void down_body(const DownArgs& a, int tile, int grp, float* red) {
  DownTile<WT, NT, LPR, CO, LISTED, LDSL> D;
  D.setup(a, tile, grp, true);
  if constexpr (LDSL != 0 && SFNN_DOWN_BATCHES) {
    D.run(a, true);
    D.loop_batches(a);
  } else {
    if (a.rg == 1) {  // the run starts at slot 0: its first ids go out before the count is in
      D.ids01(a);
      D.run(a, true);
    } else {
      D.run(a, true);
      D.ids01(a);
    }
    D.first(a);
    // the first requests are out: the loop runs at a normal priority (in
    // launch B the tile's prologue ran at a raised one)
    __builtin_amdgcn_s_setprio(1);
    D.loop(a);
  }
  D.finish(a, red, true);
}

// Host side: tile width (lanes per row), tile count, row groups and tokens
// per pass for rows of this type and length, aiming at about `items` work
// items (tiles * row groups); the arguments of an FFN's down projection.
struct DownShape {
  int lpr, tiles, rg, nt;
};
DownShape down_shape(int wt, int d, int batch, int items);
hipError_t launch_down_sum(const DownArgs& a, hipStream_t s);  // rg > 1: the partial rows into y
DownArgs ffn_down_args(const FfnLaunch& p);

}  // namespace sfnn
