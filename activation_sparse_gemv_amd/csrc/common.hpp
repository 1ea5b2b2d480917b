// Device helpers shared by the sfnn kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

namespace sfnn {

enum { WT_F32 = 0, WT_F16 = 1, WT_I4 = 2 };
enum { ACT_RELU = 0, ACT_REGLU = 1 };

constexpr int kWave = 64;

template <typename T>
__device__ __forceinline__ T bitcast(uint32_t u) { return __builtin_bit_cast(T, u); }

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Weight rows are read once per call: stream them past the caches.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(bitcast<f16x2>(a), bitcast<f16x2>(b), c, false);
}

// ---- matrix cores -----------------------------------------------------------
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// D = A B + C on one 16x16x32 fp16 tile, fp32 accumulation.  Lane l holds 8
// consecutive K values of row l % 16 of A and of column l % 16 of B (K block
// l / 16); D row 4 (l / 16) + q, column l % 16 sits in register q.
__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                0, 0);
}

// Eight fp32 values as two fp16 planes, hi = fp16(v) and lo = fp16(v - hi):
// 22 of fp32's 24 significant bits, exact for integers below 2^22 (|v| must
// stay within fp16's range: callers scale v by range_scale first).
// Power-of-two range scaling for the two-plane split.  A token whose largest
// |value| is m is carried as v * 2^-e with e = range_exp(m), which puts m in
// [2^14, 2^15): no plane overflows fp16, and the low plane stays clear of
// fp16's subnormals for every value within 2^-11 of m, so each value keeps
// its 22 bits relative to the token's largest.  The products are multiplied by
// 2^e afterwards; both steps are exact (powers of two) unless fp32 itself
// under- or overflows.  m = 0 and non-finite m leave the values unscaled.
__device__ __forceinline__ int range_exp(float m) {
  const uint32_t b = __builtin_bit_cast(uint32_t, m) & 0x7fffffffu;
  const int ef = (int)(b >> 23);
  if (b == 0u || ef == 0xff) return 0;
  const int e = (ef == 0 ? 1 : ef) - 126 - 15;  // m = f 2^k, f in [0.5, 1), k = ef - 126
  return e < -100 ? -100 : e;
}

// s_hm[t] = max(s_hm[t], hmax[st][t]) over the 32-slot steps st0 <= st <
// st1 of a [steps][32] array of non-negative floats (compared as their bit
// patterns, which order like the values), shared by a 512-thread workgroup,
// four loads in flight per thread (indices past the end re-read the last).
__device__ __forceinline__ void token_max_steps(const float* hmax, int st0, int st1, uint32_t* s_hm) {
  const int n = (st1 - st0) * 32;
  const float* base = hmax + (size_t)st0 * 32;
  for (int i0 = threadIdx.x; i0 < n; i0 += 4 * 512) {
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = i0 + 512 * j;
      v[j] = base[i < n ? i : n - 1];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = i0 + 512 * j;
      atomicMax(&s_hm[(i < n ? i : n - 1) & 31], __builtin_bit_cast(uint32_t, v[j]));
    }
  }
}

// 2^e in fp32 for e in [-126, 127].
__device__ __forceinline__ float pow2f(int e) {
  e = e < -126 ? -126 : (e > 127 ? 127 : e);
  return __builtin_bit_cast(float, (uint32_t)(e + 127) << 23);
}

__device__ __forceinline__ void split_hi_lo(const f32x4 a, const f32x4 b, u32x4& hi, u32x4& lo) {
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t h[4], l[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const f16 h0 = (f16)v[2 * k], h1 = (f16)v[2 * k + 1];
    const f16 l0 = (f16)(v[2 * k] - (float)h0), l1 = (f16)(v[2 * k + 1] - (float)h1);
    h[k] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
    l[k] = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
  }
  hi = u32x4{h[0], h[1], h[2], h[3]};
  lo = u32x4{l[0], l[1], l[2], l[3]};
}

// ---- cross-lane sums on the DPP path --------------------------------------
// Data-parallel-primitive modifiers move values between lanes inside a VALU
// instruction, with no LDS round trip (a shuffle through ds_bpermute costs an
// LDS latency per step).  Controls used (CDNA): row_shr:n = 0x110 + n and
// row_ror:n = 0x120 + n act within rows of 16 lanes; row_bcast:15 = 0x142
// feeds lane 15 of each row to the next row, row_bcast:31 = 0x143 feeds lane
// 31 to rows 2 and 3.  Lanes with no source, and rows left out by the row
// mask, read 0.  All 64 lanes must be active.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xf, false);
}
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, dpp_i<CTRL, ROWS>(__builtin_bit_cast(int, v)));
}

// Inclusive prefix sum over the 64 lanes (Hillis-Steele within rows, then
// the row totals carried across rows).
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += dpp_i<0x111>(x);
  x += dpp_i<0x112>(x);
  x += dpp_i<0x114>(x);
  x += dpp_i<0x118>(x);
  x += dpp_i<0x142, 0xa>(x);
  x += dpp_i<0x143, 0xc>(x);
  return x;
}

// Sum over the 64 lanes, returned in every lane (the scan's last lane).
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0x111>(v);
  v += dpp_f<0x112>(v);
  v += dpp_f<0x114>(v);
  v += dpp_f<0x118>(v);
  v += dpp_f<0x142, 0xa>(v);
  v += dpp_f<0x143, 0xc>(v);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), kWave - 1));
}

// Sum over each row of 16 lanes, in every lane of the row (rotations).
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0x128>(v);
  v += dpp_f<0x124>(v);
  v += dpp_f<0x122>(v);
  v += dpp_f<0x121>(v);
  return v;
}

// Sum over aligned groups of G consecutive lanes (G = 16 or 64), in every
// lane of the group.  Called with all lanes active.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(G == 16 || G == kWave, "group_sum: 16 or 64 lanes");
  if constexpr (G == kWave)
    return wave_sum(v);
  else
    return row16_sum(v);
}

// Number of set bits of m below this lane (m is wave-uniform).
__device__ __forceinline__ int bits_below_lane(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

// Stage tokens [tok0, tok0+nt) of x [*, K] into LDS xs [NT][K] (rows of
// tokens >= nt are zero) in two parts, so that loads issued later (weight
// rows) can be in flight while the activations arrive: issue() starts the
// loads of the first SP * blockDim 16-byte vectors into registers, commit()
// writes them to LDS and stages any remainder with stage-as-you-go loads.
// PERM8 applies the INT4 pairing order inside every 8-element vector.
// K * sizeof(XT) must be a multiple of 16.  Vector loads return in
// order, so waiting for these (issued first) does not wait for later loads.
template <typename XT, bool PERM8, int SP>
struct StageSplit {
  u32x4 v[SP];

  // Nothing looks at the values before commit(), so the loads stay in flight
  // while the caller issues more.  Slots past the rows load nothing (zeros):
  // redundant loads of one shared address would serialise in the cache.
  // Token of flat vector e < NT * vpr without a division (NT <= 8 is a
  // compile-time constant at every call site).
  static __device__ __forceinline__ int tok_of(int e, int vpr, int NT) {
    int t = 0;
#pragma unroll
    for (int m = 1; m < 8; ++m) t += (m < NT && e >= m * vpr) ? 1 : 0;
    return t;
  }

  __device__ __forceinline__ void issue(const XT* __restrict__ x, int K, int tok0, int nt, int NT) {
    const int vpr = K * (int)sizeof(XT) / 16;
    const int total = NT * vpr;
    const u32x4* src = reinterpret_cast<const u32x4*>(x);
#pragma unroll
    for (int j = 0; j < SP; ++j) {
      const int e = threadIdx.x + j * blockDim.x;
      const int t = tok_of(e, vpr, NT);
      v[j] = u32x4{0u, 0u, 0u, 0u};
      if (e < total && t < nt) v[j] = src[(size_t)(tok0 + t) * vpr + (e - t * vpr)];
    }
  }

  __device__ __forceinline__ void commit(XT* xs, const XT* __restrict__ x, int K, int tok0, int nt, int NT) {
    const int vpr = K * (int)sizeof(XT) / 16;
    const int total = NT * vpr;
    u32x4* dst = reinterpret_cast<u32x4*>(xs);
#pragma unroll
    for (int j = 0; j < SP; ++j) {
      const int e = threadIdx.x + j * blockDim.x;
      if (e < total) dst[e] = PERM8 ? perm8(v[j]) : v[j];  // tokens >= nt stage zeros
    }
    const u32x4* src = reinterpret_cast<const u32x4*>(x);
    for (int e = threadIdx.x + SP * blockDim.x; e < total; e += blockDim.x) {
      const int t = tok_of(e, vpr, NT);
      const u32x4 w = (t < nt) ? src[(size_t)(tok0 + t) * vpr + (e - t * vpr)] : u32x4{0u, 0u, 0u, 0u};
      dst[e] = PERM8 ? perm8(w) : w;
    }
  }

  // (x0x1, x2x3, x4x5, x6x7) -> (x0x4, x1x5, x2x6, x3x7): the INT4 pairing order
  static __device__ __forceinline__ u32x4 perm8(const u32x4 a) {
    u32x4 o;
    o.x = (a.x & 0xFFFFu) | (a.z << 16);
    o.y = (a.x >> 16) | (a.z & 0xFFFF0000u);
    o.z = (a.y & 0xFFFFu) | (a.w << 16);
    o.w = (a.y >> 16) | (a.w & 0xFFFF0000u);
    return o;
  }
};

// ---- one 16-byte weight vector against NT token rows of staged x ----------
// xs points at element (vector start) of token 0; xstride is the LDS row
// stride in elements.

// fp32 weights (4 elements) x fp32 activations.
template <int NT>
__device__ __forceinline__ void vec_f32(const u32x4 w, const float* xs, int xstride, float* acc) {
  const float w0 = bitcast<float>(w.x), w1 = bitcast<float>(w.y);
  const float w2 = bitcast<float>(w.z), w3 = bitcast<float>(w.w);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const f32x4 xv = *reinterpret_cast<const f32x4*>(xs + t * xstride);
    float a = acc[t];
    a = __builtin_fmaf(w0, xv.x, a);
    a = __builtin_fmaf(w1, xv.y, a);
    a = __builtin_fmaf(w2, xv.z, a);
    a = __builtin_fmaf(w3, xv.w, a);
    acc[t] = a;
  }
}

// fp16 weights (8 elements) x fp16 activations, fp32 accumulation.
template <int NT>
__device__ __forceinline__ void vec_f16(const u32x4 w, const f16* xs, int xstride, float* acc) {
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const u32x4 xv = *reinterpret_cast<const u32x4*>(xs + t * xstride);
    float a = acc[t];
    a = dot2(w.x, xv.x, a);
    a = dot2(w.y, xv.y, a);
    a = dot2(w.z, xv.z, a);
    a = dot2(w.w, xv.w, a);
    acc[t] = a;
  }
}

// fp16 weights (8 elements) x fp32 activations (the predictor's second stage).
template <int NT>
__device__ __forceinline__ void vec_f16_f32x(const u32x4 w, const float* xs, int xstride, float* acc) {
  float wf[8];
  const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const f16x2 h = bitcast<f16x2>(ww[k]);
    wf[2 * k] = (float)h.x;
    wf[2 * k + 1] = (float)h.y;
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const f32x4 xa = *reinterpret_cast<const f32x4*>(xs + t * xstride);
    const f32x4 xb = *reinterpret_cast<const f32x4*>(xs + t * xstride + 4);
    float a = acc[t];
    a = __builtin_fmaf(wf[0], xa.x, a);
    a = __builtin_fmaf(wf[1], xa.y, a);
    a = __builtin_fmaf(wf[2], xa.z, a);
    a = __builtin_fmaf(wf[3], xa.w, a);
    a = __builtin_fmaf(wf[4], xb.x, a);
    a = __builtin_fmaf(wf[5], xb.y, a);
    a = __builtin_fmaf(wf[6], xb.z, a);
    a = __builtin_fmaf(wf[7], xb.w, a);
    acc[t] = a;
  }
}

// INT4 weights (32 elements, one 128-group scale) x fp16 activations staged
// in the INT4 pairing order.  The nibbles enter the dot products as fp16
// subnormals, with no conversion: in offset binary (t ^ 8 = t + 8 = n), a
// nibble masked in place in bits 0-3 of a half is the fp16 value n 2^-24, and
// in bits 4-7 it is 16 n 2^-24, so two masks of the dword and two of it
// shifted by 8 give its eight nibbles as four pairs, (n0,n4) (n2,n6) at 2^-24
// and (n1,n5) (n3,n7) at 2^-20.  Every product is exact in fp32; the pairs
// are summed at their own scale and brought to 2^-24 together.  m8 holds -8
// times the sum of the same 32 activations (the offset's share, one value per
// token, stride mstride), so
//   acc += scale * (2^24 sum(n x) - 8 sum(x)) = scale * sum(t x).
template <int NT>
__device__ __forceinline__ void vec_i4(const u32x4 w, float scale, const f16* xs, const float* m8, int xstride,
                                       int mstride, float* acc) {
  const uint32_t v[4] = {w.x ^ 0x88888888u, w.y ^ 0x88888888u, w.z ^ 0x88888888u, w.w ^ 0x88888888u};
  uint32_t e[4][2], o[4][2];  // per dword: (n0,n4) (n2,n6) and 16 (n1,n5) 16 (n3,n7)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t sh = v[j] >> 8;
    e[j][0] = v[j] & 0x000F000Fu;
    o[j][0] = v[j] & 0x00F000F0u;
    e[j][1] = sh & 0x000F000Fu;
    o[j][1] = sh & 0x00F000F0u;
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float de = 0.0f, dd = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4 xv = *reinterpret_cast<const u32x4*>(xs + t * xstride + 8 * j);  // (x0,x4) (x1,x5) (x2,x6) (x3,x7)
      de = dot2(e[j][0], xv.x, de);
      dd = dot2(o[j][0], xv.y, dd);
      de = dot2(e[j][1], xv.z, de);
      dd = dot2(o[j][1], xv.w, dd);
    }
    const float sn = __builtin_fmaf(dd, 0.0625f, de);  // sum(n x) 2^-24
    acc[t] = __builtin_fmaf(scale, __builtin_fmaf(sn, 16777216.0f, m8[t * mstride]), acc[t]);
  }
}

// Elements per 16-byte weight vector.
template <int WT>
constexpr int vec_elems() { return WT == WT_F32 ? 4 : (WT == WT_F16 ? 8 : 32); }

// One batch of a weight row's 16-byte vectors held in registers.  Lane li of
// an LPR-lane group takes vectors v0, v0 + LPR, ..., v0 + (UB-1) LPR with
// v0 = li + k UB LPR.  issue() starts every load of the batch before any is
// used, so a caller can issue the batch, stage activations in LDS while the
// loads are in flight, and only then consume().  A vector past the row end
// re-reads vector v0 of the same row (in bounds) and is zeroed by a select at
// use, so the batch has no branches between its loads.  Requires v0 < nvec.
template <int WT, int LPR, int UB>
struct RowLoads {
  u32x4 w[UB];
  float sc[UB];

  // INT4: the scales go out first, so that a wait for them (the compiler may
  // convert them early) never covers this batch's weight loads
  __device__ __forceinline__ void issue(const uint8_t* __restrict__ row, const f16* __restrict__ srow, int nvec,
                                        int v0) {
    if constexpr (WT == WT_I4) {
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const int v = v0 + u * LPR;
        sc[u] = (float)srow[(v < nvec ? v : v0) >> 2];  // one scale per 4 vectors (128 elements)
      }
    }
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int v = v0 + u * LPR;
      w[u] = ld16_stream(row + 16 * (size_t)(v < nvec ? v : v0));
    }
  }

  // acc[t] += (this batch of the row) . (staged row t of xs); XT is the staged type.
  // INT4: m8 / mstride as vec_i4 takes them (per 32-element vector of the row).
  // vb: v0 of the wavefront's first lane when LPR is the wavefront (its
  // vectors are then v0 .. v0 + 63), else -1; vectors that no lane of the
  // wavefront holds are skipped by a uniform branch (no load sits in it).
  template <int NT, typename XT>
  __device__ __forceinline__ void consume(int nvec, int v0, const XT* xs, int xstride, float* acc,
                                          const float* m8 = nullptr, int mstride = 0, int vb = -1) const {
    constexpr int E = vec_elems<WT>();
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      if (vb >= 0 && vb + u * LPR >= nvec) break;
      const int v = v0 + u * LPR;
      const bool ok = v < nvec;
      // a slot past the row uses vector 0 of the staged rows (finite values)
      // and zero weights / a zero scale, so it adds exactly zero; v0 itself
      // can lie past a short row.  (INT4 needs only the zero scale: the
      // re-read weights of a row are finite.)
      const int vc = ok ? v : 0;
      const u32x4 z = {0u, 0u, 0u, 0u};
      const u32x4 wv = (WT == WT_I4 || ok) ? w[u] : z;
      if constexpr (WT == WT_F32) {
        vec_f32<NT>(wv, reinterpret_cast<const float*>(xs) + E * vc, xstride, acc);
      } else if constexpr (WT == WT_F16) {
        if constexpr (sizeof(XT) == 4)
          vec_f16_f32x<NT>(wv, reinterpret_cast<const float*>(xs) + E * vc, xstride, acc);
        else
          vec_f16<NT>(wv, reinterpret_cast<const f16*>(xs) + E * vc, xstride, acc);
      } else {
        vec_i4<NT>(wv, ok ? sc[u] : 0.0f, reinterpret_cast<const f16*>(xs) + E * vc, m8 + vc, xstride, mstride, acc);
      }
    }
  }
};

// Whole-row partial dot products: acc[t] += row . xs[t] over this lane's
// vectors.  `first` says whether the first batch (v0 = li) was already issued
// into L by the caller.
template <int WT, int LPR, int UB, int NT, typename XT>
__device__ __forceinline__ void row_dot(RowLoads<WT, LPR, UB>& L, bool first, const uint8_t* __restrict__ row,
                                        const f16* __restrict__ srow, int nvec, int li, const XT* xs, int xstride,
                                        float* acc) {
  for (int v0 = li; v0 < nvec; v0 += UB * LPR) {
    if (!(first && v0 == li)) L.issue(row, srow, nvec, v0);
    __builtin_amdgcn_sched_barrier(0);  // keep the whole batch of loads ahead of the math
    L.template consume<NT>(nvec, v0, xs, xstride, acc);
  }
}

template <typename XT>
__device__ __forceinline__ float load_as_float(const void* p, int i) {
  return (float)reinterpret_cast<const XT*>(p)[i];
}

// Mask word vb of the dense hot prefix: its 64 neurons are taken for every
// token without reading their predictor rows or thresholds; the logits read
// +inf.  Any workgroup size that is a multiple of 64 threads.
__device__ __forceinline__ void pred2_hot_word(uint64_t* mask, uint64_t* union_mask, float* logits, int f,
                                               int tok0, int nt, int vb) {
  const int lane = threadIdx.x & (kWave - 1);
  const int nw = blockDim.x / kWave;
  for (int t = threadIdx.x / kWave; t < nt; t += nw) {
    if (lane == 0) mask[(size_t)(tok0 + t) * (f / 64) + vb] = ~0ull;
    if (logits) logits[(size_t)(tok0 + t) * f + vb * 64 + lane] = __builtin_inff();
  }
  if (threadIdx.x == 0) union_mask[vb] = ~0ull;
}

// Slots s0 .. s0 + N - 1 of the union's ascending neuron list, and |U|, from
// the union mask words um[0 .. words) (words <= 1024), for a workgroup of 512
// threads: each thread takes two words; popcounts, a workgroup prefix sum (a
// lane scan per wavefront, the 8 wavefront totals through LDS), then the
// threads whose words hold ranks in [s0, s0 + N) write those neuron ids to
// ids[rank - s0]; ids past |U| stay -1.  ids: N ints of LDS, s_wt: 8.  Every
// thread calls it; on return ids and the count are the whole workgroup's.
// (The FFN's compaction inside its first matrix-core kernel: no separate
// compaction launch between the predictor and the FFN.)
template <int N>
__device__ __forceinline__ int union_window(const uint64_t* __restrict__ um, int words, int s0, int* ids, int* s_wt) {
  static_assert(N <= 512, "one id per thread at most");
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int w0 = 2 * tid;
  const uint64_t a0 = w0 < words ? um[w0] : 0ull;
  const uint64_t a1 = w0 + 1 < words ? um[w0 + 1] : 0ull;
  const int c0 = __popcll(a0), c = c0 + __popcll(a1);
  int incl = c;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  if (lane == kWave - 1) s_wt[wave] = incl;
  if (tid < N) ids[tid] = -1;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const int v = s_wt[w];
    before += w < wave ? v : 0;
    total += v;
  }
  const int r0 = before + incl - c;  // rank of a0's lowest set bit
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint64_t word = h ? a1 : a0;
    int rank = h ? r0 + c0 : r0;
    if (rank < s0 + N && rank + __popcll(word) > s0) {
      while (word && rank < s0 + N) {
        if (rank >= s0) ids[rank - s0] = 64 * (w0 + h) + __builtin_ctzll(word);
        ++rank;
        word &= word - 1;
      }
    }
  }
  __syncthreads();
  return total;
}

}  // namespace sfnn
