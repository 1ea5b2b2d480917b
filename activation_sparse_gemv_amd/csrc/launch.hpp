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
// ---- predictor ------------------------------------------------------------

// Input of the predictor's first stage.  Plain: x [B][d] as given.  Residual
// chain (r_in != null): the layer input is made in the kernel's prologue,
//     x = r_in / sqrt(mean(r_in^2) + eps)  (rounded to x's type),
// and workgroup 0 also writes it to x_out.
struct NormIn {
  const float* r_in = nullptr;  // [B][d]
  void* x_out = nullptr;        // [B][d]
  float eps = 1e-6f;
};

struct PredLaunch {
  int wt;            // WT_F32 | WT_F16
  int d, f, r;
  const void* w1_t;  // [r][d]
  const void* w2_t;  // [f][r]
  const float* tau;  // [f]
  const void* x;     // [B][d] (plain input)
  NormIn norm;       // residual-chain input when norm.r_in != null
  int batch;
  float* z;          // [B][r] workspace
  float* zpart = nullptr;  // fp16: [kPred1MaxSplits][B][r] workspace for the matrix-core stage 1
  uint64_t* mask;    // [B][f/64]
  uint64_t* union_mask;  // [f/64] OR of the batch's masks (always written)
  float* logits;     // [B][f] or null
  int hot = 0;       // leading mask words taken for every token (dense hot prefix)
};
hipError_t launch_predict(const PredLaunch& p, hipStream_t s);
// Token-group size the predictor uses for this shape (power of two <= kMaxNT).
int pred_group(int wt, int d, int r, int batch, bool chain);

// ---- FFN ------------------------------------------------------------------

enum { SRC_IDS = 0, SRC_UNION = 1, SRC_DENSE = 2 };

struct FfnLaunch {
  int wt, act;
  int d, f;
  const void *w_up, *w_gate, *w_down_t;
  const void *s_up, *s_gate, *s_down_t;
  const void *b_up, *b_gate, *b_down;
  const void* x;          // [B][d]
  int batch;
  int src;                // SRC_IDS: ids/count given; SRC_UNION: compact union_mask in the FFN kernel; SRC_DENSE
  const int32_t* ids;     // SRC_IDS
  const int32_t* count;   // SRC_IDS
  const uint64_t* union_mask;  // SRC_UNION: [f/64]
  int32_t* ids_out;       // SRC_UNION: compacted ids are written here ([f], first count valid)
  int32_t* count_out;     // SRC_UNION
  const uint64_t* mask;   // per-token gate [B][f/64] or null
  float* hrow = nullptr;  // per-row path: h [B][f] fp32 workspace (slot order), up -> down
  float* partial;         // [kMfmaPartRows][B][d] workspace: matrix-core partial rows, per-row down row groups
  int groups;             // up-projection workgroups of the per-row path
  float* y;               // [B][d] or null
  const float* r_in;      // residual add: r_out = r_in + y (both null to skip)
  float* r_out;
  void* hbuf = nullptr;   // matrix-core path: h of one 32-token pass, fp32 [32][f]
  float* hmax = nullptr;  // matrix-core path: largest |h| per 32-slot step and token, [f / 32][32]
  int32_t* sidbuf = nullptr;  // matrix-core path: slot ids [f]
  int mfma_min_batch = 0;     // matrix-core path from this batch on (0: default, < 0: never)
};
hipError_t launch_ffn(const FfnLaunch& p, hipStream_t s);

// Batches at or above these sizes run the fp16 and INT4 FFNs on the matrix
// cores (k_up_mfma + k_down_mfma, or their INT4 forms, + k_sum) unless the
// descriptor says otherwise.  The per-row INT4 kernels hold only two tokens
// per pass at d_model 12288, so from three tokens the matrix cores take half
// the time (up to two, the stack's fused look-ahead launches keep the per-row
// kernels); for fp16 the two paths cross near eight.
constexpr int kMfmaMinBatchDefault = 8;
constexpr int kMfmaMinBatchI4Default = 3;
bool ffn_uses_mfma(const FfnLaunch& p);
int mfma_groups(int d, int max_groups);  // partial rows per token on that path
// Partial rows per token the workspace holds for the matrix-core FFN (and
// for the row groups of the per-row down projection).
constexpr int kMfmaPartRows = 32;
// Per-row down projection: most row groups per tile (partial rows per token,
// at most kMfmaPartRows).
constexpr int kDownMaxGroups = 16;
// Work items (tiles x row groups) a stand-alone down launch aims at: over
// every row (dense) about three 512-thread workgroups per CU; over a listed
// subset one per CU, and only where the whole list could bring a narrow tile
// more than kDownRowGroupBytes (else one row group of narrow tiles, no
// partial rows, no sum launch).
constexpr int kDownItemsDense = 768;
constexpr int kDownItemsListed = 256;
constexpr size_t kDownRowGroupBytes = (size_t)1 << 20;
hipError_t launch_ffn_mfma(const FfnLaunch& p, hipStream_t s);
// Slots of one slot group the INT4 down kernel stages in LDS (ids and
// scales); launch_ffn_mfma refuses a shape whose groups would hold more.
constexpr int kMfmaI4MaxGroupSlots = 8192;
// INT4 passes of that path (h in the workspace as fp32 [32][f]).
// union_mask: the union compacted inside the up kernel (ids / count then the
// launch's ids_out / count_out), else null.
void mfma_all_i4(const FfnLaunch& p, const int32_t* ids, const int32_t* count, int kg, hipStream_t s,
                 const uint64_t* union_mask);
int ffn_groups(int d, int f);
// The fixed-order sum of `rows` partial rows per token (p.partial) into y
// and / or the residual add, with b_down.
hipError_t launch_sum(const FfnLaunch& p, int rows, hipStream_t s);
// Batches at or above this size run the fp16 predictor on the matrix cores
// (k_pred1_mfma + k_pred2_mfma, up to 32 tokens per pass).
constexpr int kPredMfmaMinBatch = 8;
// Stage 1 on the matrix cores splits d_model into at most this many slices
// (more workgroups than the r / 16 row tiles), added in a fixed order.
constexpr int kPred1MaxSplits = 8;
bool pred_uses_mfma(const PredLaunch& p);
hipError_t launch_pred1_mfma(const PredLaunch& p, hipStream_t s);  // residual chain: RMSNorm launch first
hipError_t launch_pred2_mfma(const PredLaunch& p, hipStream_t s);
// Predictor stages on their own (the look-ahead stack runs them apart).
hipError_t launch_predict_stage1(const PredLaunch& p, hipStream_t s);
hipError_t launch_predict_stage2(const PredLaunch& p, hipStream_t s);

// One decode step through a stack with the look-ahead predictor: layer l's
// FFN uses the mask that layer l's predictor made from the previous layer's
// input (layer 0 from its own).  pred / ffn: per-layer launch descriptors
// whose mask, union, ids, count, z, x, y and partial pointers are set; r:
// n_layers + 1 residual rows (r[0] the input, r[n_layers] the output);
// rtmp: one scratch residual row set [B][d].  dense: NULL, or per layer
// nonzero where the layer runs dense (no predictor; ffn[l] is then the dense
// launch with no mask or union).
hipError_t launch_stack_lookahead(const PredLaunch* pred, const FfnLaunch* ffn, const float* const* r,
                                  int n_layers, float eps, float* rtmp, const char* dense, hipStream_t s);

// ---- input-sparse GEMV -------------------------------------------------------

struct IsgLaunch {
  int wt;                 // WT_F32 | WT_F16 (w_t, x and bias)
  int n_in, n_out;
  const void* w_t;        // [n_in][n_out]
  const void* bias;       // [n_out] or null
  const void* x;          // [B][n_in]
  int batch;
  bool listed = false;    // ids / count already hold the inputs to read: no nonzero scan
  uint64_t* mask;         // [n_in/64] workspace: inputs nonzero for some token
  int32_t* ids;           // [n_in] the listed inputs
  int32_t* count;         // [1]
  float* partial;         // [groups][B][n_out] workspace
  int groups;             // row groups (= partial rows per token)
  float* y;               // [B][n_out]
  void* hbuf = nullptr;   // matrix-core path: [32][n_in] fp32 (x at the listed inputs)
  int32_t* sidbuf = nullptr;  // matrix-core path: [n_in] slot -> input
};
hipError_t launch_isg(const IsgLaunch& p, hipStream_t s);


// ---- head-gated attention projections ----------------------------------------

struct HeadQkvLaunch {
  int wt;                      // WT_F32 | WT_F16 (weights, biases and x)
  int d, H, hd;
  const void* w_qkv;           // [3 H hd][d]
  const void* b_qkv;           // [3 H hd] or null
  const void* x;               // [B][d]
  int batch;
  const uint64_t* head_mask;   // [B][ceil(H/64)]
  float* out;                  // [B][3 H hd]
};
hipError_t launch_head_qkv(const HeadQkvLaunch& p, hipStream_t s);
// out[t][j] = attn[t][j] if head j / hd is on for token t, else 0 ([B][H hd], x's type);
// ids / count: the rows of the heads some token uses, ascending, and how many
hipError_t launch_head_gate(int wt, const void* attn, int batch, int H, int hd, const uint64_t* head_mask,
                            void* out, int32_t* ids, int32_t* count, hipStream_t s);
int isg_groups(int n_out, int max_groups);
// fp16 inputs from this batch size on run on the matrix cores (the listed
// rows' products through k_down_mfma); the IsgLaunch then needs hbuf / sidbuf.
constexpr int kIsgMfmaMinBatch = 4;
// partial[kg][B][d] over the rows sid[0 .. count) of the fp16 matrix w_t
// [f][d], with h of one pass of up to 32 tokens as two fp16 planes [2][32][f]
// (k_down_mfma; kg = mfma_groups(d, ...)).
void launch_rows_mfma(const void* w_t, const int32_t* sid, const int32_t* count, const void* h, float* partial, int d,
                      int f, int B, int tok0, int nt, int kg, hipStream_t s);

hipError_t launch_compact(const uint64_t* mask, int batch, int f, int32_t* ids, int32_t* count,
                          uint64_t* union_mask, hipStream_t s);
hipError_t launch_fire_counts(const uint64_t* masks, int n, int f, uint32_t* counts, hipStream_t s);
hipError_t launch_gather_rows(const void* src, const int32_t* perm, int n, int64_t row_bytes, void* dst,
                              hipStream_t s);
hipError_t launch_residual_rmsnorm(const float* r_in, const float* y, float* r_out, int batch, int d,
                                   float eps, void* x_out, int xtype, hipStream_t s);
// all-ones masks, identity ids, count = f (a layer that ran dense); null pointers skipped
hipError_t launch_fill_dense(uint64_t* mask, size_t mask_words, int32_t* ids, int id_rows, int f, int32_t* count,
                             int count_n, hipStream_t s);
hipError_t launch_probe_read(const void* buf, size_t bytes, float* sink, hipStream_t s);
hipError_t launch_probe_copy(const void* src, void* dst, size_t bytes, hipStream_t s);

}  // namespace sfnn
