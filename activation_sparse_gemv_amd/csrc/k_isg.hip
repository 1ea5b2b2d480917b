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
//   k_isg        workgroup = 2048 output columns x one group of the listed
//                rows; each thread owns 8 consecutive columns (one 16-byte
//                load per fp16 row, two per fp32 row) and adds x_b[j] times
//                them over its group's rows, 16 rows of loads in flight (8
//                with more than two tokens); one fp32 partial row per row
//                group and token;
//   k_sum        bias + the row groups' partials in a fixed order.
// fp16 inputs from kIsgMfmaMinBatch tokens on take the matrix cores instead of
// k_isg: k_isg_gather lays the listed inputs' x out as the h operand of the
// FFN's down-projection kernel (k_down_mfma), which multiplies them with the
// listed rows of w_t, up to 32 tokens per pass.
// No atomics: the result is run-to-run bitwise deterministic.
#include "common.hpp"
#include "launch.hpp"

namespace sfnn {

struct IsgArgs {
  const void* w_t;       // [n_in][n_out]
  const void* x;         // [B][n_in]
  const int32_t* ids;    // listed inputs, ascending
  const int32_t* count;  // how many
  float* partial;        // [G][B][n_out]
  int n_in, n_out, B, tok0, nt, G;
};

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

template <typename XT>
__device__ __forceinline__ void isg_row(const XT* row, u32x4 (&v)[sizeof(XT) / 2]) {
#pragma unroll
  for (int h = 0; h < (int)sizeof(XT) / 2; ++h) v[h] = ld16_stream(reinterpret_cast<const uint8_t*>(row) + 16 * h);
}

// acc[t][c] += xv[t] * (8 weights of the row held in v)
template <typename XT, int NT>
__device__ __forceinline__ void isg_fma(const u32x4 (&v)[sizeof(XT) / 2], const float (&xv)[NT],
                                        float (&acc)[NT][8]) {
  float w[8];
  if constexpr (sizeof(XT) == 4) {
    const uint32_t u[8] = {v[0].x, v[0].y, v[0].z, v[0].w, v[1].x, v[1].y, v[1].z, v[1].w};
#pragma unroll
    for (int c = 0; c < 8; ++c) w[c] = bitcast<float>(u[c]);
  } else {
    const uint32_t u[4] = {v[0].x, v[0].y, v[0].z, v[0].w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f16x2 h = bitcast<f16x2>(u[c]);
      w[2 * c] = (float)h.x;
      w[2 * c + 1] = (float)h.y;
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[t][c] = __builtin_fmaf(xv[t], w[c], acc[t][c]);
}

constexpr int kIsgCols = 8 * 256;  // output columns per workgroup

// Rows whose loads are in flight together (registers: fewer with more tokens).
template <int NT>
constexpr int isg_batch() { return NT <= 2 ? 16 : 8; }

template <typename XT, int NT>
__global__ __launch_bounds__(256) void k_isg(IsgArgs a) {
  const int CB = (a.n_out + kIsgCols - 1) / kIsgCols;
  const int cb = blockIdx.x % CB, g = blockIdx.x / CB;
  const int col = cb * kIsgCols + 8 * threadIdx.x;
  const bool live = col < a.n_out;  // n_out is a multiple of 128: a thread's 8 columns are all in or all out
  const int colc = live ? col : 0;
  int cnt = *a.count;
  cnt = cnt < 0 ? 0 : (cnt > a.n_in ? a.n_in : cnt);
  const int per = (cnt + a.G - 1) / a.G;
  const int s0 = g * per;
  const int s1 = s0 + per < cnt ? s0 + per : cnt;
  const XT* w = reinterpret_cast<const XT*>(a.w_t);
  const XT* x = reinterpret_cast<const XT*>(a.x);
  float acc[NT][8];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[t][c] = 0.0f;

  constexpr int RB = isg_batch<NT>();
  // a batch of rows: every load issued before any product (rows past the
  // group re-read its last row and add nothing); the next batch's row ids are
  // fetched while this batch's rows are in flight
  int jn[RB];
  auto fetch_ids = [&](int sb) {
#pragma unroll
    for (int k = 0; k < RB; ++k) jn[k] = a.ids[sb + k < s1 ? sb + k : (s1 > 0 ? s1 - 1 : 0)];
  };
  if (s0 < s1) fetch_ids(s0);
  for (int sb = s0; sb < s1; sb += RB) {
    u32x4 v[RB][sizeof(XT) / 2];
    float xv[RB][NT];
#pragma unroll
    for (int k = 0; k < RB; ++k) {
      int j = jn[k];
      const bool ok = sb + k < s1 && j >= 0 && j < a.n_in;
      j = (j >= 0 && j < a.n_in) ? j : 0;  // past the group: the group's last listed row, times 0
      isg_row<XT>(w + (size_t)j * a.n_out + colc, v[k]);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float xx = (float)x[(size_t)(a.tok0 + (t < a.nt ? t : 0)) * a.n_in + j];
        xv[k][t] = (ok && t < a.nt) ? xx : 0.0f;
      }
    }
    if (sb + RB < s1) fetch_ids(sb + RB);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < RB; ++k) isg_fma<XT, NT>(v[k], xv[k], acc);
  }
  if (!live) return;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (t >= a.nt) break;
    float* dst = a.partial + ((size_t)g * a.B + a.tok0 + t) * a.n_out + col;
    reinterpret_cast<f32x4*>(dst)[0] = f32x4{acc[t][0], acc[t][1], acc[t][2], acc[t][3]};
    reinterpret_cast<f32x4*>(dst)[1] = f32x4{acc[t][4], acc[t][5], acc[t][6], acc[t][7]};
  }
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

int isg_groups(int n_out, int max_groups) {
  const int cb = (n_out + kIsgCols - 1) / kIsgCols;
  int g = (512 + cb - 1) / cb;  // about 512 workgroups: two per CU keep more rows in flight
  if (g > max_groups) g = max_groups;
  return g < 1 ? 1 : g;
}

template <typename XT, int NT>
static void isg_pass(const IsgLaunch& p, int tok0, int nt, hipStream_t s) {
  IsgArgs a;
  a.w_t = p.w_t;
  a.x = p.x;
  a.ids = p.ids;
  a.count = p.count;
  a.partial = p.partial;
  a.n_in = p.n_in;
  a.n_out = p.n_out;
  a.B = p.batch;
  a.tok0 = tok0;
  a.nt = nt;
  a.G = p.groups;
  const int cb = (p.n_out + kIsgCols - 1) / kIsgCols;
  hipLaunchKernelGGL((k_isg<XT, NT>), dim3(cb * p.groups), dim3(256), 0, s, a);
}

template <typename XT>
static void isg_all(const IsgLaunch& p, hipStream_t s) {
  for (int tok0 = 0; tok0 < p.batch; tok0 += kMaxNT) {
    const int nt = p.batch - tok0 < kMaxNT ? p.batch - tok0 : kMaxNT;
    if (nt == 1)
      isg_pass<XT, 1>(p, tok0, nt, s);
    else if (nt == 2)
      isg_pass<XT, 2>(p, tok0, nt, s);
    else if (nt <= 4)
      isg_pass<XT, 4>(p, tok0, nt, s);
    else
      isg_pass<XT, 8>(p, tok0, nt, s);
  }
}

hipError_t launch_isg(const IsgLaunch& p, hipStream_t s) {
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
  } else if (p.wt == WT_F32) {
    isg_all<float>(p, s);
  } else {
    isg_all<f16>(p, s);
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

}  // namespace sfnn
