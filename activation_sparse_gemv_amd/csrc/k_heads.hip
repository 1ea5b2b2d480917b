// Head-gated attention projections ([53ai] 如何充分利用结构化稀疏进行加速 and
// 验证上下文稀疏存在: contextual sparsity also covers attention heads; the
// heads an input uses are predicted and the others are skipped, up to 80% of
// them).  The attention itself (scores, softmax, values) lies outside this
// library; these are the two weight-streaming projections around it.
//
//   k_head_qkv   workgroup = 8 consecutive rows of W_qkv (4 wavefronts x 2
//                rows; head_dim is a multiple of 8, so the 8 rows belong to
//                one head) x a group of NT tokens.  The token groups of one
//                row block run on one XCD, next to each other in the grid, so
//                the second group onwards finds the rows in that XCD's L2.  A workgroup whose head is
//                off for all its tokens writes zeros and reads no weight.
//                Otherwise x is staged in LDS, in chunks of d_model that keep
//                the group's x within 64 KB, and each wavefront streams its two
//                rows chunk by chunk with 16-byte loads, kHeadUB vectors per
//                lane per row in flight, fp32 accumulation, one wavefront
//                reduction per row and token; a token whose head is off gets 0.
//   k_head_gate  x'[t][j] = attn[t][j] if head j / hd is on for token t, else
//                0.  The output projection is then the input-sparse GEMV of
//                x' (W_o^T stored input-major) over the rows of the heads some
//                token uses: workgroup 0 also lists those rows in ascending
//                order (heads flagged per thread, ballot scan in head order),
//                so the GEMV needs no nonzero scan and no compaction launch.
//
// Each sum is taken in a fixed order: results are bitwise deterministic.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace sfnn {
namespace {

constexpr int kHeadRows = 8;  // rows of W_qkv per workgroup
constexpr int kHeadUB = 4;    // 16-byte vectors per lane per row in flight

// x vectors per token staged in LDS at a time: NT tokens fill at most 64 KB.
template <int NT>
__host__ __device__ constexpr int head_chunk(int nvec) {
  return nvec < 4096 / NT ? nvec : 4096 / NT;
}

struct HeadQkvArgs {
  const uint8_t* w;       // [n][d]
  const void* b;          // [n] or null (x's type)
  const void* x;          // [B][d]
  const uint64_t* hmask;  // [B][words]
  float* out;             // [B][n]
  int d, n, H, hd, B, words;
};

template <int WT, int NT>
__global__ __launch_bounds__(256) void k_head_qkv(HeadQkvArgs a) {
  using XT = typename std::conditional<WT == WT_F32, float, f16>::type;
  extern __shared__ __align__(16) unsigned char smem[];
  XT* xs = reinterpret_cast<XT*>(smem);
  // linear block b: XCD b % 8; row block = 8 (b / 8 / NG) + b % 8, token
  // group (b / 8) % NG
  const int NG = (a.B + NT - 1) / NT;
  const int rest = blockIdx.x / 8;
  const int rb = (rest / NG) * 8 + blockIdx.x % 8;
  if (rb >= a.n / kHeadRows) return;  // padding of the last 8 row blocks
  const int row0 = rb * kHeadRows;
  const int tok0 = (rest % NG) * NT;
  const int nt = a.B - tok0 < NT ? a.B - tok0 : NT;
  const int head = (row0 % (a.H * a.hd)) / a.hd;
  bool on[NT];
  bool any = false;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    on[t] = false;
    if (t < nt) on[t] = (a.hmask[(size_t)(tok0 + t) * a.words + (head >> 6)] >> (head & 63)) & 1ull;
    any = any || on[t];
  }
  if (!any) {  // uniform over the workgroup: no weight is read
    const int t = threadIdx.x / kHeadRows, r = threadIdx.x % kHeadRows;
    if (t < nt) a.out[(size_t)(tok0 + t) * a.n + row0 + r] = 0.0f;
    return;
  }

  constexpr int E = WT == WT_F32 ? 4 : 8;  // elements per 16-byte vector
  const int nvec = a.d * (int)sizeof(XT) / 16;
  const int cvec = head_chunk<NT>(nvec);   // x vectors per token staged at a time
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int r0 = row0 + 2 * wave;
  const uint8_t* wr0 = a.w + (size_t)r0 * nvec * 16;
  const uint8_t* wr1 = wr0 + (size_t)nvec * 16;
  float acc0[NT], acc1[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc0[t] = acc1[t] = 0.0f;
  for (int c0 = 0; c0 < nvec; c0 += cvec) {  // d_model in chunks of cvec vectors
    const int cn = nvec - c0 < cvec ? nvec - c0 : cvec;
    if (c0) __syncthreads();  // every wavefront is done with the previous chunk
    for (int i = threadIdx.x; i < nt * cn; i += blockDim.x) {
      const int t = i / cn, v = i - t * cn;
      reinterpret_cast<u32x4*>(xs)[t * cvec + v] =
          ld16(reinterpret_cast<const uint8_t*>(a.x) + ((size_t)(tok0 + t) * nvec + c0 + v) * 16);
    }
    __syncthreads();
    for (int v0 = lane; v0 < cn; v0 += kHeadUB * kWave) {
      u32x4 w0[kHeadUB], w1[kHeadUB];
#pragma unroll
      for (int u = 0; u < kHeadUB; ++u) {
        const int v = v0 + u * kWave;
        const int vc = c0 + (v < cn ? v : 0);  // lanes past the chunk re-read its first vector
        w0[u] = ld16_stream(wr0 + 16 * (size_t)vc);
        w1[u] = ld16_stream(wr1 + 16 * (size_t)vc);
      }
      __builtin_amdgcn_sched_barrier(0);  // both rows' loads go out before any math
#pragma unroll
      for (int u = 0; u < kHeadUB; ++u) {
        const int v = v0 + u * kWave;
        if (v < cn) {
          if constexpr (WT == WT_F32) {
            vec_f32<NT>(w0[u], reinterpret_cast<const float*>(xs) + E * v, cvec * E, acc0);
            vec_f32<NT>(w1[u], reinterpret_cast<const float*>(xs) + E * v, cvec * E, acc1);
          } else {
            vec_f16<NT>(w0[u], reinterpret_cast<const f16*>(xs) + E * v, cvec * E, acc0);
            vec_f16<NT>(w1[u], reinterpret_cast<const f16*>(xs) + E * v, cvec * E, acc1);
          }
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    acc0[t] = group_sum<kWave>(acc0[t]);
    acc1[t] = group_sum<kWave>(acc1[t]);
  }
  if (lane == 0) {
    const float b0 = a.b ? load_as_float<XT>(a.b, r0) : 0.0f;
    const float b1 = a.b ? load_as_float<XT>(a.b, r0 + 1) : 0.0f;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t < nt) {
        float* o = a.out + (size_t)(tok0 + t) * a.n + r0;
        o[0] = on[t] ? acc0[t] + b0 : 0.0f;
        o[1] = on[t] ? acc1[t] + b1 : 0.0f;
      }
    }
  }
}

// One thread per 16-byte vector of attn ([B][H hd] in x's type); workgroup 0
// then writes the rows of the used heads to ids and their number to count.
template <int WT>
__global__ __launch_bounds__(256) void k_head_gate(const u32x4* __restrict__ attn, int B, int H, int hd,
                                                   const uint64_t* __restrict__ hmask, int words,
                                                   u32x4* __restrict__ out, int32_t* __restrict__ ids,
                                                   int32_t* __restrict__ count) {
  constexpr int E = WT == WT_F32 ? 4 : 8;
  const int nvec_row = H * hd / E, hd_vec = hd / E;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < B * nvec_row) {
    const int t = i / nvec_row, head = (i - t * nvec_row) / hd_vec;
    const bool on = (hmask[(size_t)t * words + (head >> 6)] >> (head & 63)) & 1ull;
    out[i] = on ? attn[i] : u32x4{0u, 0u, 0u, 0u};
  }
  if (blockIdx.x != 0) return;  // uniform: the list below is workgroup 0's alone
  __shared__ int wsum[4];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  int base = 0;
  for (int h0 = 0; h0 < H; h0 += 256) {  // 256 heads per round, in head order
    const int h = h0 + threadIdx.x;
    bool used = false;
    if (h < H)
      for (int t = 0; t < B; ++t) used = used || ((hmask[(size_t)t * words + (h >> 6)] >> (h & 63)) & 1ull);
    const unsigned long long bal = __ballot(used);
    const int below = __popcll(bal & ((1ull << lane) - 1ull));
    __syncthreads();  // the previous round's totals have been read
    if (lane == 0) wsum[wave] = __popcll(bal);
    __syncthreads();
    int pos = base + below;
    for (int w = 0; w < wave; ++w) pos += wsum[w];
    if (used)
      for (int r = 0; r < hd; ++r) ids[(size_t)pos * hd + r] = h * hd + r;
    base += wsum[0] + wsum[1] + wsum[2] + wsum[3];
  }
  if (threadIdx.x == 0) *count = base * hd;
}

// Token group: up to 8 tokens share each pass over the rows (x is staged in
// chunks of d_model, so any d_model fits); each group re-reads the rows.
int head_group(int batch) {
  int nt = 8;
  while (nt > 1 && nt / 2 >= batch) nt /= 2;
  return nt;
}

template <int WT, int NT>
void qkv_launch(const HeadQkvArgs& a, hipStream_t s) {
  const int nvec = a.d * (WT == WT_F32 ? 4 : 2) / 16;
  const size_t sh = (size_t)NT * head_chunk<NT>(nvec) * 16;
  const int nrb8 = (a.n / kHeadRows + 7) / 8 * 8;  // row blocks, padded to whole XCD rounds
  const dim3 grid(nrb8 * ((a.B + NT - 1) / NT));
  hipLaunchKernelGGL((k_head_qkv<WT, NT>), grid, dim3(256), sh, s, a);
}

template <int WT>
void qkv_dispatch(const HeadQkvArgs& a, int nt, hipStream_t s) {
  if (nt == 8)
    qkv_launch<WT, 8>(a, s);
  else if (nt == 4)
    qkv_launch<WT, 4>(a, s);
  else if (nt == 2)
    qkv_launch<WT, 2>(a, s);
  else
    qkv_launch<WT, 1>(a, s);
}

}  // namespace

hipError_t launch_head_qkv(const HeadQkvLaunch& p, hipStream_t s) {
  HeadQkvArgs a;
  a.w = (const uint8_t*)p.w_qkv;
  a.b = p.b_qkv;
  a.x = p.x;
  a.hmask = p.head_mask;
  a.out = p.out;
  a.d = p.d;
  a.H = p.H;
  a.hd = p.hd;
  a.n = 3 * p.H * p.hd;
  a.B = p.batch;
  a.words = (p.H + 63) / 64;
  const int nt = head_group(p.batch);
  if (p.wt == WT_F32)
    qkv_dispatch<WT_F32>(a, nt, s);
  else
    qkv_dispatch<WT_F16>(a, nt, s);
  return hipGetLastError();
}

hipError_t launch_head_gate(int wt, const void* attn, int batch, int H, int hd, const uint64_t* head_mask,
                            void* out, int32_t* ids, int32_t* count, hipStream_t s) {
  const int E = wt == WT_F32 ? 4 : 8;
  const int n = batch * (H * hd / E);
  const dim3 grid((n + 255) / 256);
  if (wt == WT_F32)
    hipLaunchKernelGGL(k_head_gate<WT_F32>, grid, dim3(256), 0, s, (const u32x4*)attn, batch, H, hd, head_mask,
                       (H + 63) / 64, (u32x4*)out, ids, count);
  else
    hipLaunchKernelGGL(k_head_gate<WT_F16>, grid, dim3(256), 0, s, (const u32x4*)attn, batch, H, hd, head_mask,
                       (H + 63) / 64, (u32x4*)out, ids, count);
  return hipGetLastError();
}

}  // namespace sfnn
