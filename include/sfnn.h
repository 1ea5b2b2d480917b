/*
 * sfnn.h -- predictor-gated activation-sparse FFN for MI355X (gfx950).
 *
 * One decode step of one FFN layer, as the pages describe it:
 *   1. a small per-layer predictor says which FFN neurons will fire
 *      (53ai.com sparsity survey, PowerInfer section "自适应稀疏预测器",
 *      adaptive sparse predictor; the hexiedandong.com PowerInfer repost:
 *      a small routing module per layer predicts the neurons an input fires);
 *   2. the predicted neurons are collected (53ai.com survey, "单层计算优化",
 *      the one-layer example where neurons 3, 4 and 5 are predicted);
 *   3. only those neurons' rows of W_up (and W_gate) and columns of W_down are
 *      read and multiplied (53ai.com survey, "激活稀疏": a zero activation zeroes
 *      the whole row it multiplies, so that row need not be loaded).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every array argument is a DEVICE pointer owned by the caller; the library
 *    allocates nothing and never reads a device value back to the host (no
 *    implicit synchronisation; calls can be captured in a HIP graph).  Its only
 *    state is sfnn_layer_noalloc's per-GPU scratch array (see there); every
 *    other call keeps none.  Descriptor structs are host memory, read during
 *    the call.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Every call is asynchronous on it and uses the caller's current device.
 *  - Arguments are validated on the host before anything is launched; a bad
 *    argument returns an error status and launches nothing.  SFNN_E_HIP means a
 *    launch failed (hipGetLastError).  Faults inside kernels surface at the
 *    caller's next synchronisation.
 *  - Shapes: d_ff % 64 == 0, d_model % 128 == 0, rank % 8 == 0,
 *    8 <= rank <= 2048, 1 <= batch <= 64, d_ff <= 65536, d_model <= 16384.  Every pointer must be
 *    16-byte aligned (SFNN_E_ALIGN), except count pointers (int32, 4-byte aligned).
 *  - Weight layout is neuron-major: W_up, W_gate and W_down^T are
 *    [d_ff][d_model] row-major, so neuron i owns one contiguous row of each
 *    (row i of W_down^T is column i of the conventional W_down[d_model][d_ff]).
 *  - Activations x: [batch][d_model] row-major, fp32 when the weights are
 *    SFNN_F32, else fp16.  Outputs y: [batch][d_model] fp32.
 *  - Masks: [batch][d_ff/64] uint64, neuron i is bit (i % 64) of word i / 64
 *    (LSB first).
 *  - SFNN_I4G128: weights are two's-complement INT4, element 2k in the low
 *    nibble of byte k of the row ([d_ff][d_model/2] uint8), with one fp16
 *    scale per row and 128 consecutive elements ([d_ff][d_model/128]);
 *    w = q * s (the weight-only scheme of the ciyundata.com survey, section
 *    2.2 量化, dequantised inside the kernel).
 */
#ifndef SFNN_H
#define SFNN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SFNN_OK = 0,
  SFNN_E_NULL = 1,      /* a required pointer is NULL                        */
  SFNN_E_SHAPE = 2,     /* a size is outside the limits listed above         */
  SFNN_E_ALIGN = 3,     /* a pointer is not 16-byte aligned                  */
  SFNN_E_DTYPE = 4,     /* unknown or inconsistent weight / activation types */
  SFNN_E_WORKSPACE = 5, /* workspace smaller than sfnn_workspace_bytes()     */
  SFNN_E_HIP = 6        /* a HIP launch reported an error                    */
} sfnn_status;

typedef enum { SFNN_F32 = 0, SFNN_F16 = 1, SFNN_I4G128 = 2 } sfnn_wtype;
typedef enum { SFNN_RELU = 0, SFNN_REGLU = 1 } sfnn_act;

/* Per-layer low-rank predictor.  logit = W2^T (W1^T x); neuron i is predicted
 * active iff logit_i > tau_i (strict).  wtype is SFNN_F32 or SFNN_F16 and
 * must match the activation type of x.  An F16 predictor called with 8 or
 * more tokens runs on the matrix cores (fp32 accumulation, z carried as two
 * fp16 parts: 22 significant bits, |z| within fp16's range); smaller batches
 * and F32 predictors take the per-row kernels.
 *
 * Dense hot prefix.  With the neurons in hot-first order (sfnn_fire_counts,
 * sfnn_hot_first_perm, sfnn_gather_rows: [53ai] PowerInfer 概述 and
 * 单层计算优化, hot neurons are found offline and carry most activations)
 * the first hot_prefix neurons (a multiple of 64, at most d_ff; 0 turns it
 * off) are taken for every token without reading their W2^T rows or tau:
 * their mask bits are set, their logits (when asked for) read +inf, and the
 * FFN computes them for every token, so their own ReLU / ReGLU decides their
 * share exactly.  This saves their rank * element-size predictor bytes per
 * neuron; it pays when the union of the batch fires them nearly always.
 * Outside [0, d_ff] or not a multiple of 64: SFNN_E_SHAPE.
 *
 * Dense switch (sfnn_layer, sfnn_layer_noalloc, sfnn_stack_decode).  The
 * sparse path pays off while the batch's union of active neurons stays a
 * small share of d_ff (DejaVu's contextual sparsity is per token; the union
 * of B tokens grows with B, and past a crossover the gathered rows cost more
 * than reading the matrices whole: 53ai.com sparsity survey, DejaVu section).
 * From batch >= dense_min_batch on (a positive value; 0, the default, and
 * negative values never switch) these calls skip the predictor and run the
 * dense FFN: every neuron for every token, its own ReLU / ReGLU deciding its
 * share, which is the masked FFN under an all-ones mask.  They then report
 * that mask (all bits set), ids 0..d_ff-1 and count = d_ff.  The stack reads
 * each layer's own field, so one step may mix sparse and dense layers.  How
 * fast the union grows depends on how the layer's neurons fire: under a
 * power law it stays far below d_ff at batches where uniform firing fills it
 * (same page, throughput paragraph), so there is no default threshold;
 * sfnn_dense_min_batch derives one from profiled fire counts.  The field is
 * read per call. */
typedef struct sfnn_pred {
  int32_t d_model, d_ff, rank;
  int32_t wtype;       /* sfnn_wtype: F32 or F16                         */
  const void* w1_t;    /* [rank][d_model]                                */
  const void* w2_t;    /* [d_ff][rank] (rows below hot_prefix unread)    */
  const float* tau;    /* [d_ff]       (entries below hot_prefix unread) */
  int32_t hot_prefix;  /* dense hot prefix, see above; 0: none           */
  int32_t dense_min_batch; /* dense switch, see above; <= 0: never       */
} sfnn_pred;

/* One FFN layer.  ReLU:  y = b_down + sum_i relu(W_up[i].x + b_up[i]) W_down[:, i]
 *                ReGLU: y = b_down + sum_i relu(W_gate[i].x + b_gate[i])
 *                                         * (W_up[i].x + b_up[i]) W_down[:, i]
 * Biases have x's type (fp32 for F32 weights, else fp16); NULL means zero.
 *
 * Batch-aware dispatch (sparse, dense, layer and stack calls).  Gathering
 * rows is the pages' per-row kernel (PowerInfer's neuron-aware operators,
 * [53ai] GPU-CPU混合执行); once a batch has many tokens the work over the union
 * of active rows is a dense contraction.  An F16 or I4G128 FFN called with
 * batch >= mfma_min_batch (0 selects the default: 8 for F16, 3 for I4G128,
 * whose per-row kernels hold only a few tokens per pass; a negative value
 * never) runs it on the matrix cores: the up projection over the gathered
 * rows and the down projection over column slices, fp32 accumulation, h
 * carried between them in fp32 and entering the down products as two fp16
 * parts of h times a per-token power of two (22 significant bits relative to
 * the token's largest |h|, no overflow at any finite |h|), the partial rows
 * added in a fixed order
 * (deterministic, no atomics).  I4G128 nibbles enter as exact fp16 integers
 * and the group scales are applied in fp32, so no weight is rounded.  Smaller
 * batches and F32 weights take the per-row kernels.  The field is read per
 * call, like the rest of the descriptor. */
typedef struct sfnn_ffn {
  int32_t d_model, d_ff;
  int32_t wtype;       /* sfnn_wtype                                     */
  int32_t act;         /* sfnn_act                                       */
  const void* w_up;    /* [d_ff][d_model]  (I4G128: [d_ff][d_model/2])   */
  const void* w_gate;  /* ReGLU only, same layout; NULL for ReLU         */
  const void* w_down_t;/* [d_ff][d_model]  (I4G128: [d_ff][d_model/2])   */
  const void* s_up;    /* I4G128 only: fp16 [d_ff][d_model/128]          */
  const void* s_gate;
  const void* s_down_t;
  const void* b_up;    /* [d_ff]     or NULL                             */
  const void* b_gate;  /* [d_ff]     or NULL                             */
  const void* b_down;  /* [d_model]  or NULL                             */
  int32_t mfma_min_batch; /* batch-aware dispatch, see below; 0: default */
} sfnn_ffn;

/* Bytes of device workspace needed by sfnn_predict / sfnn_sparse_ffn /
 * sfnn_dense_ffn / sfnn_layer for this layer and batch (either descriptor may
 * be NULL when only the other's calls are used).  0 on invalid input.  The
 * workspace needs no initialisation and may be reused by the next call on the
 * same stream. */
size_t sfnn_workspace_bytes(const sfnn_pred* pred, const sfnn_ffn* ffn, int32_t batch);

/* Predictor (steps 1 of the header comment).  Writes mask [batch][d_ff/64]
 * and, if logits != NULL, the fp32 logits [batch][d_ff].  The mask equals
 * (logits > tau) evaluated on those fp32 logits. */
sfnn_status sfnn_predict(const sfnn_pred* pred, const void* x, int32_t batch,
                         uint64_t* mask, float* logits,
                         void* ws, size_t ws_bytes, void* stream);

/* Compaction (step 2): union U of the batch's masks, ids[0..count) = the set
 * bits of U in ascending order, *count = |U| (device int32).  Entries of ids
 * past count are left untouched.  union_mask [d_ff/64] is written if not NULL.
 * ids must have room for d_ff entries. */
sfnn_status sfnn_compact(const uint64_t* mask, int32_t batch, int32_t d_ff,
                         int32_t* ids, int32_t* count, uint64_t* union_mask,
                         void* stream);

/* Sparse FFN (step 3) over the neurons ids[0..*count) (ascending, unique,
 * < d_ff; entries >= d_ff are skipped and *count is clamped to d_ff).  ids
 * must have room for d_ff entries, as sfnn_compact writes them: entries past
 * *count may be read (and are never used), so the kernels need not wait for
 * the count before reading the list.
 * If mask != NULL each token b only takes neuron i when bit i of mask[b] is
 * set (a select, not a multiply); with mask == NULL every token takes every
 * listed neuron.  Writes y [batch][d_model] fp32. */
sfnn_status sfnn_sparse_ffn(const sfnn_ffn* ffn, const void* x, int32_t batch,
                            const int32_t* ids, const int32_t* count,
                            const uint64_t* mask, float* y,
                            void* ws, size_t ws_bytes, void* stream);

/* The same FFN over all d_ff neurons with no gather: the dense baseline. */
sfnn_status sfnn_dense_ffn(const sfnn_ffn* ffn, const void* x, int32_t batch, float* y,
                           void* ws, size_t ws_bytes, void* stream);

/* predict -> compact -> sparse_ffn for one layer (same results as the three
 * calls in sequence; the compaction runs inside the FFN's first kernel).
 * mask/ids/count are outputs the caller may inspect; any of them may be NULL,
 * then they live in ws.  With batch > 1 every token is gated by its own mask.
 * pred and ffn must agree on d_model, d_ff and the activation type.  From
 * batch >= pred->dense_min_batch on the layer runs dense (see sfnn_pred). */
sfnn_status sfnn_layer(const sfnn_pred* pred, const sfnn_ffn* ffn, const void* x,
                       int32_t batch, float* y, uint64_t* mask, int32_t* ids,
                       int32_t* count, void* ws, size_t ws_bytes, void* stream);

/* sfnn_layer for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, and harnesses that forbid hipMalloc.
 * Same arguments, results and execution rules as sfnn_layer, without ws /
 * ws_bytes: the workspace is a library-owned device array of
 * SFNN_NOALLOC_SCRATCH_BYTES on each GPU the library runs on, held until the
 * process ends.  The call allocates nothing (no hipMalloc / hipFree, no
 * allocating library routine).
 *  - Returns SFNN_E_WORKSPACE, before touching the GPU, when
 *    sfnn_workspace_bytes(pred, ffn, batch) exceeds SFNN_NOALLOC_SCRATCH_BYTES.
 *  - The first call on a device looks up that device's copy of the array
 *    (SFNN_E_HIP if the lookup fails).
 *  - Every call on one GPU shares that GPU's array, which keeps the last
 *    call's contents (nothing in it needs to start at zero).  Calls that
 *    overlap on one GPU (two streams, or two host threads) race on it and
 *    give wrong results: serialise them. */
#define SFNN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
sfnn_status sfnn_layer_noalloc(const sfnn_pred* pred, const sfnn_ffn* ffn, const void* x,
                               int32_t batch, float* y, uint64_t* mask, int32_t* ids,
                               int32_t* count, void* stream);

/* One decode step through a stack of n_layers FFN layers joined by the
 * pre-norm residual chain without gain (the pages give no stack recipe; this
 * is the plain reading of "RMS-normalised inputs"):
 *     r_0 = r_in;  for l = 0..n_layers-1:
 *         x_l = r_l / sqrt(mean(r_l^2) + eps)   (rounded to x's type)
 *         m_l = layer l's predicted mask (see flags)
 *         y_l = layer l's FFN over the union of m_l, each token gated by its
 *               own mask, exactly as sfnn_sparse_ffn computes it
 *         r_{l+1} = r_l + y_l
 *     r_out = r_{n_layers}.
 * flags = 0: m_l = predictor_l(x_l), i.e. each layer exactly as sfnn_layer.
 * flags = SFNN_STACK_LOOKAHEAD: m_l = predictor_l(x_{l-1}) for l >= 1 (and
 *     predictor_0(x_0)): DejaVu's asynchronous look-ahead, where the next
 *     layer's sparsity is predicted one step ahead so the predictor runs
 *     beside the current layer's FFN (53ai.com sparsity survey, DejaVu
 *     section 如何充分利用结构化稀疏进行加速).
 * A layer whose preds[l].dense_min_batch is positive and <= batch runs dense
 * instead (see sfnn_pred): no predictor, m_l all ones, y_l the dense FFN.
 * preds / ffns are HOST arrays of n_layers descriptors that share one shape
 * and type (d_model, d_ff, rank, wtype, act); their device pointers may differ.
 * r_in, r_out: [batch][d_model] fp32 (r_out may alias r_in).  Optional
 * per-layer captures (NULL to skip): x_cap [n_layers][batch][d_model] in x's
 * type, y_cap [n_layers][batch][d_model] fp32, mask_cap
 * [n_layers][batch][d_ff/64] (the mask layer l used), ids_cap [n_layers][d_ff]
 * (first count valid), count_cap [n_layers].  The workspace is
 * sfnn_workspace_bytes(&preds[0], &ffns[0], batch).  Same execution rules as
 * every call: asynchronous on `stream`, no device allocation, no host
 * synchronisation (capturable in a graph). */
#define SFNN_STACK_LOOKAHEAD 1
sfnn_status sfnn_stack_decode(int32_t n_layers, const sfnn_pred* preds, const sfnn_ffn* ffns, int32_t batch,
                              const float* r_in, float* r_out, float eps, int32_t flags, void* x_cap, float* y_cap,
                              uint64_t* mask_cap, int32_t* ids_cap, int32_t* count_cap, void* ws, size_t ws_bytes,
                              void* stream);

/* Stack step between layers (pre-norm residual chain, no gain):
 * r_out = r_in + y (y may be NULL: r_out = r_in; r_out may alias r_in);
 * x_out = r_out / sqrt(mean(r_out^2) + eps) written as xtype (F32 or F16).
 * r_in, y, r_out: [batch][d_model] fp32. */
sfnn_status sfnn_residual_rmsnorm(const float* r_in, const float* y, float* r_out, int32_t batch,
                                  int32_t d_model, float eps, void* x_out, int32_t xtype, void* stream);

/* Offline profiling (hexiedandong.com PowerInfer repost, power-law paragraph:
 * neuron firing follows a power law, so hot neurons are found ahead of time).
 * counts[i] += number of the n_masks masks ([n_masks][d_ff/64]) with bit i set. */
sfnn_status sfnn_fire_counts(const uint64_t* masks, int32_t n_masks, int32_t d_ff,
                             uint32_t* counts, void* stream);

/* Hot-first order (HOST memory in and out): perm[new] = original neuron id,
 * by descending count, ties by ascending id. */
sfnn_status sfnn_hot_first_perm(const uint32_t* counts, int32_t d_ff, int32_t* perm);

/* Dense-switch threshold from a fire-count profile (HOST memory; no GPU call).
 * With p_i = counts[i] / n_profiled the fire rate of neuron i over
 * n_profiled independent tokens, a batch of b such tokens is expected to
 * touch the share u(b) = mean_i (1 - (1 - p_i)^b) of the d_ff neurons
 * (53ai.com sparsity survey, DejaVu section, throughput paragraph: the share
 * grows with the batch, sub-linearly when firing follows a power law).
 * *out = the smallest b in [1, max_batch] with u(b) >= crossover, or -1 when
 * none reaches it; crossover is the union share from which the dense FFN
 * beats predictor + sparse FFN on the target (measured per weight type).
 * Store *out in sfnn_pred.dense_min_batch.  Errors: counts or out NULL ->
 * SFNN_E_NULL; n_profiled < 1, d_ff < 1, max_batch < 1, crossover outside
 * (0, 1] or not a number, or a count above n_profiled -> SFNN_E_SHAPE
 * (*out untouched). */
sfnn_status sfnn_dense_min_batch(const uint32_t* counts, int32_t n_profiled, int32_t d_ff, float crossover,
                                 int32_t max_batch, int32_t* out);

/* dst row k = src row perm[k] for k < n_rows, rows of row_bytes bytes
 * (row_bytes % 2 == 0; applies a relayout to weights, scales and biases).
 * dst must not overlap src (an in-place relayout would race): overlapping
 * ranges return SFNN_E_SHAPE without launching. */
sfnn_status sfnn_gather_rows(const void* src, const int32_t* perm, int32_t n_rows,
                             int64_t row_bytes, void* dst, void* stream);

/* Measurement helpers: read `bytes` (multiple of 16) with 16-byte loads and
 * fold them into sink[0] (read-bandwidth probe), and copy `bytes` from src to
 * dst (reference copy for traffic counters). */
sfnn_status sfnn_probe_read(const void* buf, size_t bytes, float* sink, void* stream);
sfnn_status sfnn_probe_copy(const void* src, void* dst, size_t bytes, void* stream);

/* Input-sparse GEMV: y = bias + W x for inputs with many zero entries.
 * The relufication page's second stage ([53ai] 第二阶段——插入新的ReLU) puts a
 * ReLU after the normalisation layer, so the inputs of the projections that
 * follow it (FFN up projection, attention QKV) are sparse, and a zero input
 * selects a column of W that contributes nothing.  W is stored input-major:
 * w_t [n_in][n_out], row j the column of W that input j multiplies, so a
 * skipped input skips one contiguous row.  wtype is SFNN_F32 or SFNN_F16;
 * x [batch][n_in] and bias [n_out] (NULL: zero) have that type.
 * Limits: n_in a multiple of 64 in [64, 65536], n_out a multiple of 128 in
 * [128, 65536], 1 <= batch <= 64; pointers 16-byte aligned (count: 4). */
typedef struct sfnn_isg {
  int32_t n_in, n_out;
  int32_t wtype;       /* SFNN_F32 or SFNN_F16                           */
  const void* w_t;     /* [n_in][n_out]                                  */
  const void* bias;    /* [n_out] or NULL                                */
} sfnn_isg;

/* Device workspace bytes for sfnn_input_sparse_gemv (0 on invalid input). */
size_t sfnn_isg_workspace_bytes(const sfnn_isg* op, int32_t batch);

/* J = the inputs j with x_b[j] != 0 for some token b (ascending; -0.0 is a
 * zero, NaN is not); for every token y_b = bias + sum_{j in J} x_b[j] w_t[j, :]
 * with fp32 accumulation, so only the rows of w_t listed in J are read.  A
 * token's own zero inputs in J add exact zeros: y_b is the dense product up to
 * rounding.  Writes y [batch][n_out] fp32 and, when not NULL, cols [n_in]
 * (J, first *count entries) and count [1] on the device.  Asynchronous on the
 * stream; the result is bitwise deterministic. */
sfnn_status sfnn_input_sparse_gemv(const sfnn_isg* op, const void* x, int32_t batch, float* y,
                                   int32_t* cols, int32_t* count, void* ws, size_t ws_bytes,
                                   void* stream);

const char* sfnn_status_str(sfnn_status s);
/* Head-gated attention projections ([53ai] 如何充分利用结构化稀疏进行加速 and
 * 验证上下文稀疏存在: contextual sparsity covers attention heads as well as
 * MLP neurons; the heads each input uses are predicted and up to 80% of heads
 * are skipped).  The attention between the two projections (scores, softmax,
 * values) is the caller's.  Weights, biases, x and attn share one type (F32 or
 * F16); outputs are fp32.  head_mask: [batch][ceil(n_heads/64)] packed uint64
 * words, bit h%64 of word h/64 set when token t uses head h (the caller's
 * head predictor).  Limits: d_model as elsewhere, head_dim a multiple of 8 in
 * [8, 512], n_heads * head_dim a multiple of 64 and at most 65536. */
typedef struct sfnn_heads {
  int32_t d_model, n_heads, head_dim;
  int32_t wtype;       /* SFNN_F32 or SFNN_F16                           */
  const void* w_qkv;   /* [3 n_heads head_dim][d_model]: the q rows of all
                          heads (head h: rows h*head_dim ..), then k, then v */
  const void* b_qkv;   /* [3 n_heads head_dim] or NULL                   */
  const void* w_o_t;   /* [n_heads head_dim][d_model]: row j = column j of W_o */
  const void* b_o;     /* [d_model] or NULL                              */
} sfnn_heads;

/* qkv[t][r] = w_qkv[r] . x_t + b_qkv[r] for the rows r of heads on for token
 * t, and 0 for the rest ([batch][3 n_heads head_dim] fp32, caller-owned).
 * Rows of heads that no token of the batch uses are not read. */
sfnn_status sfnn_head_qkv(const sfnn_heads* op, const void* x, int32_t batch, const uint64_t* head_mask,
                          float* qkv, void* stream);

/* y_t = b_o + sum over heads h on for token t of attn_t[h head_dim ..
 * (h+1) head_dim) . w_o_t[the same rows] ([batch][d_model] fp32).  attn:
 * [batch][n_heads head_dim]; the entries of heads off for a token are not
 * used (may hold anything).  Runs as the input-sparse GEMV of the head-masked
 * attn, so rows whose input is zero for every token, the unused heads among
 * them, are not read.  ws: sfnn_heads_workspace_bytes(op, batch) bytes. */
sfnn_status sfnn_head_out(const sfnn_heads* op, const void* attn, int32_t batch, const uint64_t* head_mask,
                          float* y, void* ws, size_t ws_bytes, void* stream);
size_t sfnn_heads_workspace_bytes(const sfnn_heads* op, int32_t batch);

int32_t sfnn_version(void);  /* 300 and up: sfnn_ffn has mfma_min_batch; 310 and up: sfnn_input_sparse_gemv; 320 and up: sfnn_pred has hot_prefix; 330 and up: sfnn_head_qkv, sfnn_head_out; 340 and up: sfnn_pred has dense_min_batch; 350 and up: sfnn_dense_min_batch, per-layer switch in the stack, no default threshold */

#ifdef __cplusplus
}
#endif
#endif /* SFNN_H */
