// Input-sparse GEMV: y = bias + W x for inputs with many zero entries
// (relufication stage 2, [53ai] 第二阶段——插入新的ReLU: a ReLU after the
// normalisation layer makes the inputs of the up and QKV projections sparse,
// and a zero input selects a column of W that contributes nothing).
//
// W is stored input-major, w_t [n_in][n_out]: the column that input j
// multiplies is one contiguous row, so skipping a zero input skips a whole
// row of HBM.  Three launches:
//   k_isg_mask   one wavefront per 64 inputs: ballot of (x_b[j] != 0) over
//                the batch, OR-ed into one mask word (a -0.0 is a zero, a NaN
//                is not);
//   k_compact    the union's set bits in ascending order (shared with the
//                FFN's compaction);
//   k_down       the FFN's column-tiled down projection (down_body.hpp)
//                over the listed rows of w_t, with x_b[j] as the coefficient
//                of row j: each workgroup owns a tile of every listed row and
//                writes y (with the bias) directly, or, where the list could
//                be long, one partial row per row group that k_sum adds in
//                a fixed order.
// Single-launch form (per-row path, n_in <= kIsgSelfMaxIn, one row group):
//   k_isg_self   every workgroup lists the rows itself, in its own LDS (one
//                ballot per 64 inputs, a popcount scan, the set bits written
//                in ascending order), then runs its k_down tile over that
//                list; workgroup 0 also writes the list and its count.  One
//                fp16 token packs its input into the list entry, so the
//                loop's only global loads are weights.
// fp16 inputs from kIsgMfmaMinBatch tokens on take the matrix cores instead of
// k_down: k_isg_gather lays the listed inputs' x out as the h operand of the
// FFN's matrix-core down-projection kernel (k_down_mfma), which multiplies
// them with the listed rows of w_t, up to 32 tokens per pass, and k_sum adds
// the slot groups' partial rows with the bias.
// No atomics: the result is run-to-run bitwise deterministic.
#include "ffn_launch.hpp"

namespace sfnn {

template <typename XT>
__global__ __launch_bounds__(256) void k_isg_mask(const XT* __restrict__ x, int batch, int n_in,
                                                  uint64_t* __restrict__ mask) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = blockIdx.x * 4 + threadIdx.x / kWave;  // mask word of this wavefront
  if (w >= n_in / 64) return;                          // whole wavefronts only
  bool nz = false;
  for (int b = 0; b < batch; ++b) nz |= (float)x[(size_t)b * n_in + 64 * w + lane] != 0.0f;
  const unsigned long long word = __ballot(nz);
  if (lane == 0) mask[w] = (uint64_t)word;
}

constexpr int kIsgCols = 8 * 256;  // output columns per 2048-column block (sizes the partial rows)

// ---- single-launch form --------------------------------------------------------

constexpr int kIsgSelfMaxIn = 16384;  // 16-bit ids, 32 KB of LDS for the list; 32 inputs per thread
constexpr int kIsgPackedMaxIn = 8192;  // one fp16 token: id | coefficient entries, 32 KB

struct SelfList {
  const void* x;            // inputs [B][n_in]: the nonzero ones are listed
  int n_in, batch;
  int32_t* cols_out;        // [n_in] or null: the list, written by workgroup 0
  int32_t* count_out;       // [1] or null
};

// The workgroup's row list in ascending order, into its dynamic LDS (count
// first, 16-bit ids after it, or PACKED: 32-bit entries id | the one token's
// fp16 input << 16); every thread of the workgroup calls it.  Thread i owns
// inputs 32 i .. 32 i + 31 (n_in <= 16384 = 512 x 32): their nonzero bits
// from independent 16-byte loads of every token, an exclusive prefix sum of
// the threads' popcounts
// (lane scan per wavefront, wavefront totals through LDS), then each thread
// writes its own entries in ascending order.
template <typename XT, bool PACKED>
__device__ __forceinline__ void isg_build_list(const SelfList& L) {
  constexpr int NW = kDownThreads / kWave;
  constexpr int E = 16 / (int)sizeof(XT);  // inputs per 16-byte vector
  constexpr int VPT = 32 / E;              // vectors per thread
  __shared__ int s_wt[NW];
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int j0 = 32 * tid;
  const bool mine = j0 < L.n_in;
  uint32_t m = 0;
  u32x4 v[PACKED ? VPT : 1];  // PACKED: the one token's inputs, kept for the entries
  if constexpr (PACKED) {
    // one fp16 token: its inputs are the coefficients
#pragma unroll
    for (int q = 0; q < VPT; ++q)
      v[q] = mine ? ld16(reinterpret_cast<const uint8_t*>(L.x) + ((size_t)j0 + q * E) * sizeof(XT))
                  : u32x4{0u, 0u, 0u, 0u};
  }
  {
    // nonzero: magnitude bits set (-0.0 is a zero, NaN is not)
    for (int t = 0; t < L.batch; ++t) {
      u32x4 w[VPT];
#pragma unroll
      for (int q = 0; q < VPT; ++q) {
        if constexpr (PACKED)
          w[q] = v[q];
        else
          w[q] = mine ? ld16(reinterpret_cast<const uint8_t*>(L.x) + ((size_t)t * L.n_in + j0 + q * E) * sizeof(XT))
                      : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int q = 0; q < VPT; ++q) {
        const uint32_t c[4] = {w[q].x, w[q].y, w[q].z, w[q].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if constexpr (sizeof(XT) == 2) {
            m |= (uint32_t)((c[k] & 0x7fffu) != 0) << (q * E + 2 * k);
            m |= (uint32_t)((c[k] & 0x7fff0000u) != 0) << (q * E + 2 * k + 1);
          } else {
            m |= (uint32_t)((c[k] & 0x7fffffffu) != 0) << (q * E + k);
          }
        }
      }
    }
  }
  // exclusive prefix of the popcounts over the workgroup
  const int c = __popc(m);
  int incl = c;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int t = __shfl_up(incl, off);
    if (lane >= off) incl += t;
  }
  if (lane == kWave - 1) s_wt[wave] = incl;
  __syncthreads();
  int pos = incl - c, total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int t = s_wt[w];
    pos += w < wave ? t : 0;
    total += t;
  }
  int* base = lds_list_base();
  if (tid == 0) base[0] = total;
  const bool report = blockIdx.x == 0 && L.cols_out;
  uint32_t mm = m;
  while (mm) {
    const int e = __builtin_ctz(mm), j = j0 + e;
    mm &= mm - 1;
    if constexpr (PACKED) {
      const uint32_t word = e < 16 ? (e < 8 ? (e < 4 ? (e < 2 ? v[0].x : v[0].y) : (e < 6 ? v[0].z : v[0].w))
                                            : (e < 12 ? (e < 10 ? v[1].x : v[1].y) : (e < 14 ? v[1].z : v[1].w)))
                                   : (e < 24 ? (e < 20 ? (e < 18 ? v[2].x : v[2].y) : (e < 22 ? v[2].z : v[2].w))
                                             : (e < 28 ? (e < 26 ? v[3].x : v[3].y) : (e < 30 ? v[3].z : v[3].w)));
      const uint32_t xb = (e & 1) ? (word >> 16) : (word & 0xffffu);
      lds_list_packed()[pos] = (uint32_t)j | (xb << 16);
    } else {
      lds_list_ids()[pos] = (uint16_t)j;
    }
    if (report) L.cols_out[pos] = j;
    ++pos;
  }
  if (blockIdx.x == 0 && tid == 0 && L.count_out) L.count_out[0] = total;
  __syncthreads();
}

template <int WT, int NT, int LPR, int CO, bool PACKED>
__global__ __launch_bounds__(kDownThreads) void k_isg_self(DownArgs a, SelfList L, int ntiles) {
  using XT = typename std::conditional<WT == WT_F32, float, f16>::type;
  __shared__ __align__(16) float red[DownRed<WT, NT, LPR>::floats];
  isg_build_list<XT, PACKED>(L);
  int tile, grp;
  down_item(blockIdx.x, ntiles, 8 / LPR, tile, grp);
  down_body<WT, NT, LPR, CO, true, PACKED ? 2 : 1>(a, tile, grp, red);
}

// Matrix-core path: the pass's x at the listed inputs in slot order as fp32
// [32][n_in] (fp16 values, so k_down_mfma's split leaves its low plane zero
// and needs no range scaling), tokens past the pass and slots past the list
// zero, and the slot -> input map (slots past the list re-read the last
// listed row), for slots below |J| rounded up to 32.
__global__ __launch_bounds__(256) void k_isg_gather(const f16* __restrict__ x, const int32_t* __restrict__ ids,
                                                    const int32_t* __restrict__ count, int n_in, int tok0, int nt,
                                                    float* __restrict__ h, int32_t* __restrict__ sid) {
  const int s = blockIdx.x * 256 + threadIdx.x;
  int cnt = *count;
  cnt = cnt < 0 ? 0 : (cnt > n_in ? n_in : cnt);
  if (s >= ((cnt + 31) & ~31) || s >= n_in) return;
  int j = s < cnt ? ids[s] : (cnt > 0 ? ids[cnt - 1] : 0);
  const bool ok = s < cnt && j >= 0 && j < n_in;
  j = j >= 0 && j < n_in ? j : 0;
  sid[s] = j;
  for (int t = 0; t < 32; ++t) h[(size_t)t * n_in + s] = (ok && t < nt) ? (float)x[(size_t)(tok0 + t) * n_in + j] : 0.0f;
}

// ---- host side ---------------------------------------------------------------

// The down-projection arguments of the per-row path: the listed rows of w_t,
// x as the coefficients.
static DownArgs isg_down_args(const IsgLaunch& p) {
  DownArgs a{};
  a.w = (const uint8_t*)p.w_t;
  a.s = nullptr;
  a.ids = p.ids;
  a.count = p.count;
  a.n_slots = p.n_in;
  a.n_rows = p.n_in;
  a.co = p.x;
  a.co_stride = p.n_in;
  a.bias = p.bias;
  a.bias_f32 = p.wt == WT_F32 ? 1 : 0;
  a.y = p.y;
  a.r_in = nullptr;
  a.r_out = nullptr;
  a.d = p.n_out;
  a.tok0 = 0;
  a.nt = p.batch;
  a.rg = 1;
  a.part = p.partial;  // at least kDownMaxGroups partial rows per token (isg_groups)
  a.batch = p.batch;
  return a;
}

// The single-launch form applies: the per-row path (not the matrix cores), a
// list that fits the LDS, and a shape whose row list needs no row groups.
#ifndef SFNN_ISG_SELF
#define SFNN_ISG_SELF 1  // 0: always the mask, compaction and GEMV launches
#endif
static bool isg_self_fits(const IsgLaunch& p) {
  if (!SFNN_ISG_SELF || p.n_in > kIsgSelfMaxIn) return false;
  if (p.wt == WT_F16 && p.batch >= kIsgMfmaMinBatch && p.hbuf && p.sidbuf) return false;
  const DownShape narrow = down_shape(p.wt, p.n_out, p.batch, 0);
  if ((size_t)p.n_in * 16 * narrow.lpr > kDownRowGroupBytes) return false;
  // LDS: the reduction buffer, the list and the scan's words within 64 KB
  const int cpl = p.wt == WT_F32 ? 4 : 8;
  const size_t red = (size_t)(kDownThreads / kWave) * 4 * narrow.lpr * narrow.nt * cpl * 4;
  const bool packed = p.wt == WT_F16 && p.batch == 1 && p.n_in <= kIsgPackedMaxIn;
  return red + 16 + (size_t)p.n_in * (packed ? 4 : 2) + 512 <= 65536;
}

template <int WT, int NT, int CO, bool PACKED = false>
static void isg_self_pass(const DownArgs& a, const SelfList& L, const DownShape& sh, hipStream_t s) {
  const dim3 grid(sh.tiles), blk(kDownThreads);
  const size_t lds = 16 + (size_t)L.n_in * (PACKED ? 4 : 2);
  switch (sh.lpr) {
    case 1: hipLaunchKernelGGL((k_isg_self<WT, NT, 1, CO, PACKED>), grid, blk, lds, s, a, L, sh.tiles); break;
    case 2: hipLaunchKernelGGL((k_isg_self<WT, NT, 2, CO, PACKED>), grid, blk, lds, s, a, L, sh.tiles); break;
    case 4: hipLaunchKernelGGL((k_isg_self<WT, NT, 4, CO, PACKED>), grid, blk, lds, s, a, L, sh.tiles); break;
    default: hipLaunchKernelGGL((k_isg_self<WT, NT, 8, CO, PACKED>), grid, blk, lds, s, a, L, sh.tiles); break;
  }
}

// Every token group of the batch; each launch lists the rows of the whole batch.
// One fp16 token with a short list: the packed entries (no coefficient loads).
// (Rows whose narrowest tiles fall under a 128-byte line were also tried in
// whole lines over row groups plus a sum launch: slower, the sum launch
// costing more than the wider tiles save at these sizes.)
template <int WT, int CO>
static void isg_self_all(DownArgs a, const SelfList& L, int batch, hipStream_t s) {
  const DownShape sh = down_shape(WT, a.d, batch, 0);
  a.rg = 1;
  if constexpr (WT == WT_F16) {
    if (batch == 1 && L.n_in <= kIsgPackedMaxIn) {
      a.tok0 = 0;
      a.nt = 1;
      isg_self_pass<WT, 1, CO, true>(a, L, sh, s);
      return;
    }
  }
  for (int tok0 = 0; tok0 < batch; tok0 += sh.nt) {
    a.tok0 = tok0;
    a.nt = batch - tok0 < sh.nt ? batch - tok0 : sh.nt;
    switch (sh.nt) {
      case 1: isg_self_pass<WT, 1, CO>(a, L, sh, s); break;
      case 2: isg_self_pass<WT, 2, CO>(a, L, sh, s); break;
      case 4: isg_self_pass<WT, 4, CO>(a, L, sh, s); break;
      default: isg_self_pass<WT, 8, CO>(a, L, sh, s); break;
    }
  }
}

static void isg_self(const IsgLaunch& p, hipStream_t s) {
  const DownArgs a = isg_down_args(p);
  SelfList L{};
  L.x = p.x;
  L.n_in = p.n_in;
  L.batch = p.batch;
  L.cols_out = p.ids;
  L.count_out = p.count;
  if (p.wt == WT_F32)
    isg_self_all<WT_F32, CO_X32>(a, L, p.batch, s);
  else
    isg_self_all<WT_F16, CO_X16>(a, L, p.batch, s);
}

int isg_groups(int n_out, int max_groups) {
  const int cb = (n_out + kIsgCols - 1) / kIsgCols;
  int g = (512 + cb - 1) / cb;  // about 512 workgroups: two per CU keep more rows in flight
  if (g > max_groups) g = max_groups;
  return g < 1 ? 1 : g;
}

// The per-row path: the column-tiled down projection over the listed rows,
// x as the coefficients.
template <int WT>
static void isg_rows(const IsgLaunch& p, hipStream_t s) {
  down_all<WT, WT == WT_F32 ? CO_X32 : CO_X16>(isg_down_args(p), p.batch, s);
}

hipError_t launch_isg(const IsgLaunch& p, hipStream_t s) {
  if (!p.listed && isg_self_fits(p)) {
    isg_self(p, s);
    return hipGetLastError();
  }
  if (!p.listed) {
    const int words = p.n_in / 64;
    if (p.wt == WT_F32)
      hipLaunchKernelGGL(k_isg_mask<float>, dim3((words + 3) / 4), dim3(256), 0, s, (const float*)p.x, p.batch,
                         p.n_in, p.mask);
    else
      hipLaunchKernelGGL(k_isg_mask<f16>, dim3((words + 3) / 4), dim3(256), 0, s, (const f16*)p.x, p.batch,
                         p.n_in, p.mask);
    const hipError_t e = launch_compact(p.mask, 1, p.n_in, p.ids, p.count, nullptr, s);
    if (e != hipSuccess) return e;
  }
  int groups = p.groups;
  if (p.wt == WT_F16 && p.batch >= kIsgMfmaMinBatch && p.hbuf && p.sidbuf) {
    groups = mfma_groups(p.n_out, p.groups);
    for (int tok0 = 0; tok0 < p.batch; tok0 += 32) {
      const int nt = p.batch - tok0 < 32 ? p.batch - tok0 : 32;
      hipLaunchKernelGGL(k_isg_gather, dim3((p.n_in + 255) / 256), dim3(256), 0, s, (const f16*)p.x, p.ids,
                         p.count, p.n_in, tok0, nt, (float*)p.hbuf, p.sidbuf);
      launch_rows_mfma(p.w_t, p.sidbuf, p.count, p.hbuf, p.partial, p.n_out, p.n_in, p.batch, tok0, nt, groups, s);
    }
    FfnLaunch f{};
    f.wt = p.wt;
    f.d = p.n_out;
    f.batch = p.batch;
    f.partial = p.partial;
    f.groups = groups;
    f.b_down = p.bias;
    f.y = p.y;
    return launch_sum(f, groups, s);
  }
  if (p.wt == WT_F32)
    isg_rows<WT_F32>(p, s);
  else
    isg_rows<WT_F16>(p, s);
  return hipGetLastError();
}

}  // namespace sfnn
