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

// The per-row path: the column-tiled down projection over the listed rows,
// x as the coefficients.
template <int WT>
static void isg_rows(const IsgLaunch& p, hipStream_t s) {
  DownArgs a;
  a.w = (const uint8_t*)p.w_t;
  a.s = nullptr;
  a.ids = p.ids;
  a.count = p.count;
  a.n_slots = p.n_in;
  a.n_rows = p.n_in;
  a.co = p.x;
  a.co_stride = p.n_in;
  a.bias = p.bias;
  a.bias_f32 = WT == WT_F32 ? 1 : 0;
  a.y = p.y;
  a.r_in = nullptr;
  a.r_out = nullptr;
  a.d = p.n_out;
  a.tok0 = 0;
  a.nt = p.batch;
  a.rg = 1;
  a.part = p.partial;  // at least kDownMaxGroups partial rows per token (isg_groups)
  a.batch = p.batch;
  down_all<WT, WT == WT_F32 ? CO_X32 : CO_X16>(a, p.batch, s);
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
