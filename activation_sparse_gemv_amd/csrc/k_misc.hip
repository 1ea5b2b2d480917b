// Mask compaction, offline fire counting, row relayout, the stack's
// residual + RMSNorm step, and two bandwidth probes.
#include <algorithm>
#include "common.hpp"
#include "launch.hpp"

namespace sfnn {

// Union of the batch's masks and the ascending list of its set bits
// (53ai.com sparsity survey, PowerInfer one-layer example 单层计算优化: only the
// predicted set {3, 4, 5} is computed).  One workgroup: every thread owns one
// mask word, a popcount + workgroup prefix sum gives each word its output
// offset, and ids come out in ascending order with no sort.  Sparse unions
// (at most 8 set bits per word on average) are emitted by each thread for its
// own word, lowest bit first; denser ones by whole words per wavefront, one
// bit per lane at the word's offset plus the set bits below the lane, so each
// word's ids go out as one coalesced store.
__global__ __launch_bounds__(1024) void k_compact(const uint64_t* __restrict__ mask, int batch, int words,
                                                  int32_t* __restrict__ ids, int32_t* __restrict__ count,
                                                  uint64_t* __restrict__ union_mask) {
  // words <= 1024 (d_ff <= 65536): thread w owns mask word w
  __shared__ int wsum[16];
  __shared__ uint64_t su[1024];
  __shared__ int so[1024];
  const int w = threadIdx.x;
  const int lane = w & (kWave - 1), wave = w / kWave;
  uint64_t u = 0;
  if (w < words)
    for (int b = 0; b < batch; ++b) u |= mask[(size_t)b * words + w];
  const int local = __popcll(u);
  const int v = wave_incl_scan(local);  // inclusive scan inside the wave
  if (lane == kWave - 1) wsum[wave] = v;
  __syncthreads();
  if (wave == 0) {
    const int nw = blockDim.x / kWave;
    const int s = wave_incl_scan(lane < nw ? wsum[lane] : 0);
    if (lane < nw) wsum[lane] = s;
  }
  __syncthreads();
  int off = v - local + (wave > 0 ? wsum[wave - 1] : 0);
  const int nwaves = blockDim.x / kWave;
  const int total = wsum[nwaves - 1];
  if (w < words && union_mask) union_mask[w] = u;
  if (w == blockDim.x - 1) *count = total;
  if (total <= 8 * words) {  // uniform over the workgroup
    if (w < words) {
      while (u) {
        ids[off++] = w * 64 + __builtin_ctzll(u);
        u &= u - 1;
      }
    }
    return;
  }
  su[w] = u;
  so[w] = off;
  __syncthreads();
#pragma unroll 4
  for (int j = wave; j < words; j += nwaves) {
    const uint64_t m = su[j];
    if ((m >> lane) & 1ull) ids[so[j] + bits_below_lane(m)] = j * 64 + lane;
  }
}

// counts[i] += number of masks with bit i set (offline hot/cold profiling).
__global__ __launch_bounds__(256) void k_fire_counts(const uint64_t* __restrict__ masks, int n, int f,
                                                     uint32_t* __restrict__ counts) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= f) return;
  const int words = f / 64;
  uint32_t c = 0;
  for (int m = 0; m < n; ++m) c += (uint32_t)((masks[(size_t)m * words + (i >> 6)] >> (i & 63)) & 1ull);
  counts[i] += c;
}

// dst row k = src row perm[k]; rows whose perm entry is out of range are left untouched.
__global__ __launch_bounds__(256) void k_gather_rows(const uint8_t* __restrict__ src,
                                                     const int32_t* __restrict__ perm, int n, int64_t row_bytes,
                                                     uint8_t* __restrict__ dst) {
  for (int k = blockIdx.x; k < n; k += gridDim.x) {
    const int sr = perm[k];
    if ((unsigned)sr >= (unsigned)n) continue;
    const uint8_t* a = src + (size_t)sr * row_bytes;
    uint8_t* b = dst + (size_t)k * row_bytes;
    if ((row_bytes & 15) == 0) {
      for (int64_t o = threadIdx.x * 16; o < row_bytes; o += blockDim.x * 16)
        *reinterpret_cast<u32x4*>(b + o) = *reinterpret_cast<const u32x4*>(a + o);
    } else {
      for (int64_t o = threadIdx.x * 2; o < row_bytes; o += blockDim.x * 2)
        *reinterpret_cast<uint16_t*>(b + o) = *reinterpret_cast<const uint16_t*>(a + o);
    }
  }
}

__device__ __forceinline__ float block_sum256(float v, float* sh) {
  v = group_sum<kWave>(v);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  const float t = ((sh[0] + sh[1]) + sh[2]) + sh[3];
  __syncthreads();
  return t;
}

// r_out = r_in + y (y and r_out optional); x = (r_in + y) / sqrt(mean((r_in + y)^2) + eps).
// One workgroup per token; each thread keeps up to 64 values in registers
// (d_model <= 16384), loaded as 16-byte vectors.
__global__ __launch_bounds__(256) void k_residual_rmsnorm(const float* r_in, const float* y, float* r_out, int d,
                                                          float eps, void* __restrict__ xo, int xtype) {
  constexpr int kMaxV = 16;  // float4 vectors per thread
  __shared__ float sh[4];
  const size_t base = (size_t)blockIdx.x * d;
  const int nv = d / 4;
  const f32x4* ri = reinterpret_cast<const f32x4*>(r_in + base);
  const f32x4* yi = reinterpret_cast<const f32x4*>(y + base);
  f32x4 v[kMaxV];
#pragma unroll
  for (int j = 0; j < kMaxV; ++j) {
    const int e = threadIdx.x + j * blockDim.x;
    v[j] = (e < nv) ? ri[e] : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if (y) {
#pragma unroll
    for (int j = 0; j < kMaxV; ++j) {
      const int e = threadIdx.x + j * blockDim.x;
      if (e < nv) v[j] += yi[e];
    }
  }
  float ss = 0.0f;
  f32x4* ro = reinterpret_cast<f32x4*>(r_out + base);
#pragma unroll
  for (int j = 0; j < kMaxV; ++j) {
    const int e = threadIdx.x + j * blockDim.x;
    if (e < nv) {
      if (r_out) ro[e] = v[j];
      ss = __builtin_fmaf(v[j].x, v[j].x, ss);
      ss = __builtin_fmaf(v[j].y, v[j].y, ss);
      ss = __builtin_fmaf(v[j].z, v[j].z, ss);
      ss = __builtin_fmaf(v[j].w, v[j].w, ss);
    }
  }
  const float tot = block_sum256(ss, sh);
  const float inv = 1.0f / __builtin_sqrtf(tot / (float)d + eps);
#pragma unroll
  for (int j = 0; j < kMaxV; ++j) {
    const int e = threadIdx.x + j * blockDim.x;
    if (e < nv) {
      const f32x4 o = v[j] * inv;
      if (xtype == WT_F32) {
        reinterpret_cast<f32x4*>(xo)[base / 4 + e] = o;
      } else {
        const f16x2 a = {(f16)o.x, (f16)o.y}, b = {(f16)o.z, (f16)o.w};
        uint2 pk;
        pk.x = __builtin_bit_cast(uint32_t, a);
        pk.y = __builtin_bit_cast(uint32_t, b);
        reinterpret_cast<uint2*>(xo)[base / 4 + e] = pk;
      }
    }
  }
}

// What a layer that ran dense reports: every mask bit set (mask_words 64-bit
// words), every id in order (id_rows rows of f ids) and count = f
// (count_n entries).  Each pointer may be null.
__global__ __launch_bounds__(256) void k_fill_dense(uint64_t* __restrict__ mask, size_t mask_words,
                                                    int32_t* __restrict__ ids, int id_rows, int f,
                                                    int32_t* __restrict__ count, int count_n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  const size_t t0 = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (mask)
    for (size_t i = t0; i < mask_words; i += stride) mask[i] = ~0ull;
  if (ids)
    for (size_t i = t0; i < (size_t)id_rows * f; i += stride) ids[i] = (int32_t)(i % (size_t)f);
  if (count)
    for (size_t i = t0; i < (size_t)count_n; i += stride) count[i] = f;
}

__global__ __launch_bounds__(256) void k_probe_read(const u32x4* __restrict__ buf, size_t nvec,
                                                    float* __restrict__ sink) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(buf + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) sink[0] = 1.0f;  // keeps the loads alive
}

__global__ __launch_bounds__(256) void k_probe_copy(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                    size_t nvec) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += stride) dst[i] = src[i];
}

hipError_t launch_compact(const uint64_t* mask, int batch, int f, int32_t* ids, int32_t* count,
                          uint64_t* union_mask, hipStream_t s) {
  hipLaunchKernelGGL(k_compact, dim3(1), dim3(1024), 0, s, mask, batch, f / 64, ids, count, union_mask);
  return hipGetLastError();
}

hipError_t launch_fire_counts(const uint64_t* masks, int n, int f, uint32_t* counts, hipStream_t s) {
  hipLaunchKernelGGL(k_fire_counts, dim3((f + 255) / 256), dim3(256), 0, s, masks, n, f, counts);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* src, const int32_t* perm, int n, int64_t row_bytes, void* dst,
                              hipStream_t s) {
  const int grid = n < 65536 ? n : 65536;
  hipLaunchKernelGGL(k_gather_rows, dim3(grid), dim3(256), 0, s, (const uint8_t*)src, perm, n, row_bytes,
                     (uint8_t*)dst);
  return hipGetLastError();
}

hipError_t launch_residual_rmsnorm(const float* r_in, const float* y, float* r_out, int batch, int d,
                                   float eps, void* x_out, int xtype, hipStream_t s) {
  hipLaunchKernelGGL(k_residual_rmsnorm, dim3(batch), dim3(256), 0, s, r_in, y, r_out, d, eps, x_out, xtype);
  return hipGetLastError();
}

hipError_t launch_fill_dense(uint64_t* mask, size_t mask_words, int32_t* ids, int id_rows, int f, int32_t* count,
                             int count_n, hipStream_t s) {
  const size_t n = std::max(mask_words, std::max((size_t)id_rows * f, (size_t)count_n));
  size_t grid = (n + 255) / 256;
  if (grid > 1024) grid = 1024;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(k_fill_dense, dim3((unsigned)grid), dim3(256), 0, s, mask, mask_words, ids, id_rows, f, count,
                     count_n);
  return hipGetLastError();
}

hipError_t launch_probe_read(const void* buf, size_t bytes, float* sink, hipStream_t s) {
  const size_t nvec = bytes / 16;
  size_t grid = (nvec + 255) / 256;
  if (grid > 4096) grid = 4096;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(k_probe_read, dim3((unsigned)grid), dim3(256), 0, s, (const u32x4*)buf, nvec, sink);
  return hipGetLastError();
}

hipError_t launch_probe_copy(const void* src, void* dst, size_t bytes, hipStream_t s) {
  const size_t nvec = bytes / 16;
  size_t grid = (nvec + 255) / 256;
  if (grid > 4096) grid = 4096;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(k_probe_copy, dim3((unsigned)grid), dim3(256), 0, s, (const u32x4*)src, (u32x4*)dst, nvec);
  return hipGetLastError();
}

}  // namespace sfnn
