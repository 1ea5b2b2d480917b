// Host-side launchers of the sfnn kernels (internal to libsfnn.so).
// Every launcher enqueues on `stream` and returns hipGetLastError().
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sfnn {

// Largest token group one kernel pass handles; bigger batches run in passes.
constexpr int kMaxNT = 8;
// LDS budget for staged activations per workgroup.
constexpr int kStageBytes = 64 * 1024;

struct PredLaunch {
  int wt;            // WT_F32 | WT_F16
  int d, f, r;
  const void* w1_t;  // [r][d]
  const void* w2_t;  // [f][r]
  const float* tau;  // [f]
  const void* x;     // [B][d]
  int batch;
  float* z;          // [B][r] workspace
  uint64_t* mask;    // [B][f/64]
  float* logits;     // [B][f] or null
};
hipError_t launch_predict(const PredLaunch& p, hipStream_t s);

struct FfnLaunch {
  int wt, act;
  int d, f;
  const void *w_up, *w_gate, *w_down_t;
  const void *s_up, *s_gate, *s_down_t;
  const void *b_up, *b_gate, *b_down;
  const void* x;          // [B][d]
  int batch;
  const int32_t* ids;     // null: dense (identity, count = f)
  const int32_t* count;
  const uint64_t* mask;   // per-token gate or null
  float* y;               // [B][d]
  float* h;               // [B][f] workspace
  float* partial;         // [R][kMaxNT][d] workspace
  int row_blocks;         // R
};
hipError_t launch_ffn(const FfnLaunch& p, hipStream_t s);
int ffn_row_blocks(int d, int f);

hipError_t launch_compact(const uint64_t* mask, int batch, int f, int32_t* ids, int32_t* count,
                          uint64_t* union_mask, hipStream_t s);
hipError_t launch_fire_counts(const uint64_t* masks, int n, int f, uint32_t* counts, hipStream_t s);
hipError_t launch_gather_rows(const void* src, const int32_t* perm, int n, int64_t row_bytes, void* dst,
                              hipStream_t s);
hipError_t launch_residual_rmsnorm(const float* r_in, const float* y, float* r_out, int batch, int d,
                                   float eps, void* x_out, int xtype, hipStream_t s);
hipError_t launch_probe_read(const void* buf, size_t bytes, float* sink, hipStream_t s);
hipError_t launch_probe_copy(const void* src, void* dst, size_t bytes, hipStream_t s);

}  // namespace sfnn
