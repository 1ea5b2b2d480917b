// Launch templates of the per-row gathered FFN, instantiated per weight type
// in k_ffn_f32.hip, k_ffn_f16.hip and k_ffn_i4.hip: k_up (the listed rows of
// W_up / W_gate -> h) then k_down (the same rows of W_down^T, column-tiled,
// -> y and the residual row).
#pragma once
#include "down_body.hpp"
#include "ffn_body.hpp"

namespace sfnn {

template <int WT, int ACT, int NT, int SRC, int NTH, int RV, int UW>
__global__ __launch_bounds__(NTH) void k_up(FfnArgs a) {
  up_body<WT, ACT, NT, SRC, NTH, RV, false, UW>(a, blockIdx.x, gridDim.x);
}

template <int WT, int NT, int LPR, int CO, bool LISTED>
__global__ __launch_bounds__(kDownThreads) void k_down(DownArgs a, int ntiles) {
  __shared__ __align__(16) float red[DownRed<WT, NT, LPR>::floats];
  int tile, grp;
  down_item(blockIdx.x, ntiles, 8 / LPR, tile, grp);
  down_body<WT, NT, LPR, CO, LISTED>(a, tile, grp, red);
}

// Union-mask words each lane holds: 4 covers d_ff <= 16384, 16 covers 65536.
inline int union_words_per_lane(int f) { return f / 64 <= 4 * kWave ? 4 : 16; }

template <int WT, int ACT, int NT>
static void up_pass(const FfnLaunch& p, int tok0, int nt, bool first, hipStream_t s) {
  using XT = typename std::conditional<WT == WT_F32, float, f16>::type;
  const FfnArgs a = ffn_args(p, tok0, nt, first);
  const size_t sh = (size_t)NT * p.d * sizeof(XT) + (WT == WT_I4 ? (size_t)NT * (p.d / 32) * 4 : 0);  // + vec_i4's m8
  const int G = p.groups;
  constexpr int NTH = 512;
  if (p.src == SRC_UNION) {
    if (union_words_per_lane(p.f) == 4)
      hipLaunchKernelGGL((k_up<WT, ACT, NT, SRC_UNION, NTH, 2, 4>), dim3(G), dim3(NTH), sh, s, a);
    else
      hipLaunchKernelGGL((k_up<WT, ACT, NT, SRC_UNION, NTH, 2, 16>), dim3(G), dim3(NTH), sh, s, a);
  } else if (p.src == SRC_IDS) {
    hipLaunchKernelGGL((k_up<WT, ACT, NT, SRC_IDS, NTH, 2, 2>), dim3(G), dim3(NTH), sh, s, a);
  } else {
    hipLaunchKernelGGL((k_up<WT, ACT, NT, SRC_DENSE, NTH, 2, 2>), dim3(G), dim3(NTH), sh, s, a);
  }
}

// One down pass over tokens [tok0, tok0 + nt) with coefficients `co`.
template <int WT, int NT, int CO, bool LISTED>
static void down_pass_l(const DownArgs& a, const DownShape& sh, hipStream_t s) {
  const dim3 grid(sh.tiles * sh.rg), blk(kDownThreads);
  switch (sh.lpr) {
    case 1: hipLaunchKernelGGL((k_down<WT, NT, 1, CO, LISTED>), grid, blk, 0, s, a, sh.tiles); break;
    case 2: hipLaunchKernelGGL((k_down<WT, NT, 2, CO, LISTED>), grid, blk, 0, s, a, sh.tiles); break;
    case 4: hipLaunchKernelGGL((k_down<WT, NT, 4, CO, LISTED>), grid, blk, 0, s, a, sh.tiles); break;
    default: hipLaunchKernelGGL((k_down<WT, NT, 8, CO, LISTED>), grid, blk, 0, s, a, sh.tiles); break;
  }
}

template <int WT, int NT, int CO>
static void down_pass(const DownArgs& a, const DownShape& sh, hipStream_t s) {
  if (a.ids)
    down_pass_l<WT, NT, CO, true>(a, sh, s);
  else if constexpr (CO == CO_H)  // gathered coefficients need a row list
    down_pass_l<WT, NT, CO, false>(a, sh, s);
}

// Every down pass of a batch (token groups of sh.nt).
template <int WT, int CO>
void down_all(DownArgs a, int batch, hipStream_t s) {
  int items = kDownItemsDense;
  if (a.ids) {
    const DownShape narrow = down_shape(WT, a.d, batch, 0);
    items = (size_t)a.n_slots * 16 * narrow.lpr > kDownRowGroupBytes ? kDownItemsListed : 0;
  }
  const DownShape sh = down_shape(WT, a.d, batch, items);
  a.rg = sh.rg;
  for (int tok0 = 0; tok0 < batch; tok0 += sh.nt) {
    a.tok0 = tok0;
    a.nt = batch - tok0 < sh.nt ? batch - tok0 : sh.nt;
    switch (sh.nt) {
      case 1: down_pass<WT, 1, CO>(a, sh, s); break;
      case 2: down_pass<WT, 2, CO>(a, sh, s); break;
      case 4:
        if constexpr (WT != WT_I4) down_pass<WT, 4, CO>(a, sh, s);
        break;
      default:
        if constexpr (WT != WT_I4) down_pass<WT, 8, CO>(a, sh, s);
        break;
    }
  }
  if (sh.rg > 1) (void)launch_down_sum(a, s);  // errors surface through hipGetLastError
}

template <int WT, int ACT>
void ffn_all(const FfnLaunch& p, hipStream_t s) {
  const FfnShape sh = ffn_shape(WT, p.d, p.batch);
  for (int tok0 = 0; tok0 < p.batch; tok0 += sh.nt) {
    const int nt = (p.batch - tok0 < sh.nt) ? (p.batch - tok0) : sh.nt;
    const bool first = tok0 == 0;
    switch (sh.nt) {
      case 1: up_pass<WT, ACT, 1>(p, tok0, nt, first, s); break;
      case 2: up_pass<WT, ACT, 2>(p, tok0, nt, first, s); break;
      case 4: up_pass<WT, ACT, 4>(p, tok0, nt, first, s); break;
      default: up_pass<WT, ACT, 8>(p, tok0, nt, first, s); break;
    }
  }
  if (p.y || p.r_out) down_all<WT, CO_H>(ffn_down_args(p), p.batch, s);
}

// One weight type's entry points (k_ffn_<type>.hip).
void ffn_run_f32(const FfnLaunch& p, hipStream_t s);
void ffn_run_f16(const FfnLaunch& p, hipStream_t s);
void ffn_run_i4(const FfnLaunch& p, hipStream_t s);

}  // namespace sfnn
