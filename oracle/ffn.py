"""Float64 CPU oracle of the predictor-gated sparse FFN.  TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may call this module.  It imports nothing from the product
package, and the product never imports it.

Pages cited (by title and section):

* [53ai] the 53ai.com survey of sparsity for 10x LLM inference on consumer
  GPUs; sections "激活稀疏" (activation sparsity), "验证上下文稀疏存在"
  (verifying contextual sparsity), "概述" and "单层计算优化" (PowerInfer
  overview and one-layer example), "自适应稀疏预测器" (adaptive sparse
  predictor), "工程效果" / "吞吐影响" (engineering effect, throughput vs batch).
* [news] the hexiedandong.com repost of the PowerInfer news article
  ("2080 Ti runs a 70B model ... 11x"): power-law paragraph, the 3/4/5
  example, INT4 paragraph.
* [ciyun] the ciyundata.com survey "LLM inference optimisation techniques",
  section 2.2 量化 (weight-only quantisation dequantised inside the kernel).
* [53ai] sections "如何充分利用结构化稀疏进行加速" and "验证上下文稀疏存在"
  (contextual sparsity covers attention heads as well as MLP neurons: a
  predictor picks the heads per input, up to 80% of heads are skipped).
* [53ai] section "第二阶段——插入新的ReLU" (relufication stage 2: a ReLU after
  the normalisation layer makes the inputs of the up and QKV projections
  sparse).

Readings of points the pages leave open (each also listed in the design notes):

* The per-layer predictor is read as a rank-r linear map z = W1^T x,
  logit = W2^T z, with no hidden nonlinearity and no bias; neuron i is
  predicted active iff logit_i > tau_i (strict).
* Masks are packed uint64 words, bit i%64 of word i/64, LSB first.
* A batch reads the union of the tokens' predicted sets; each token is gated
  by its own mask (a select: gated-off neurons contribute nothing at all).
* Dense hot prefix (opt-in, for a hot-first layout): neurons i < H are taken
  for every token without the predictor; their logits read +inf.
* INT4: element 2k in the low nibble of byte k, two's complement, one fp16
  scale per row and 128 consecutive elements; w = q * s.

Parity status: every function here is pinned by a ``-m "not gpu"`` test
(brute force, closed forms, invariants or the pages' worked example); none is
"parity unpinned".
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "unpack_mask", "pack_mask", "predict", "guard_band", "compact", "dequant_int4",
    "rows_f64", "masked_ffn", "dense_ffn", "true_active", "fire_counts",
    "hot_first_perm", "permute_layer_ids", "residual_rmsnorm", "input_sparse_gemv",
    "head_qkv", "head_out",
]

_U24 = 2.0 ** -24


# ---------------------------------------------------------------------------
# mask layout
# ---------------------------------------------------------------------------

def unpack_mask(words, f: int) -> np.ndarray:
    """[..., f/64] uint64 -> [..., f] bool, bit j of word w is neuron 64w+j."""
    words = np.asarray(words, dtype=np.uint64)
    shifts = np.arange(64, dtype=np.uint64)
    bits = (words[..., :, None] >> shifts) & np.uint64(1)
    return bits.reshape(words.shape[:-1] + (words.shape[-1] * 64,))[..., :f].astype(bool)


def pack_mask(bits) -> np.ndarray:
    """Inverse of :func:`unpack_mask` (f must be a multiple of 64)."""
    bits = np.asarray(bits, dtype=bool)
    f = bits.shape[-1]
    if f % 64:
        raise ValueError("d_ff must be a multiple of 64")
    grouped = bits.reshape(bits.shape[:-1] + (f // 64, 64)).astype(np.uint64)
    weights = np.uint64(1) << np.arange(64, dtype=np.uint64)
    return (grouped * weights).sum(axis=-1, dtype=np.uint64)


# ---------------------------------------------------------------------------
# predictor  ([53ai] 自适应稀疏预测器; [news] per-layer predicting router)
# ---------------------------------------------------------------------------

def predict(w1_t, w2_t, tau, x, hot_prefix: int = 0):
    """Low-rank predictor: logits [B][f] (float64) and the active mask [B][f].

    z_j = sum_k W1[k, j] x_k with W1^T stored as w1_t [r][d];
    logit_i = sum_j W2[j, i] z_j with W2^T stored as w2_t [f][r];
    active_i  <=>  logit_i > tau_i.

    hot_prefix H: in a hot-first layout ([53ai] PowerInfer 概述 and 单层计算优化:
    the hot neurons, found offline, carry most activations) neurons i < H are
    taken for every token without asking the predictor, so the FFN runs them
    as a dense block and their own ReLU decides what they contribute.  Their
    mask bits are set whatever tau_i holds and their logits read +inf.
    """
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    a = np.asarray(w1_t, dtype=np.float64)
    b = np.asarray(w2_t, dtype=np.float64)
    z = x @ a.T                      # [B][r]
    logits = z @ b.T                 # [B][f]
    t = np.asarray(tau, dtype=np.float64)
    active = logits > t[None, :]
    logits[:, :hot_prefix] = np.inf
    active[:, :hot_prefix] = True
    return logits, active


def guard_band(w1_t, w2_t, x) -> np.ndarray:
    """Width of the band around tau where an fp32 evaluation may flip a bit.

    For dot products evaluated in fp32 (any order, fused or not) the error is
    at most n * 2^-24 * sum |a_k b_k| (first order).  Applying that to both
    stages gives |logit_fp32 - logit| <= (d + r + 2) 2^-24 S_i with
    S_i = sum_j |W2[j, i]| sum_k |W1[k, j]| |x_k|.  Returns [B][f].
    """
    x = np.atleast_2d(np.abs(np.asarray(x, dtype=np.float64)))
    a = np.abs(np.asarray(w1_t, dtype=np.float64))
    b = np.abs(np.asarray(w2_t, dtype=np.float64))
    d, r = a.shape[1], a.shape[0]
    s = (x @ a.T) @ b.T
    return (d + r + 2) * _U24 * s


# ---------------------------------------------------------------------------
# compaction  ([53ai] 单层计算优化: only the predicted set {3,4,5} is computed)
# ---------------------------------------------------------------------------

def compact(words, batch: int, f: int):
    """Union over the batch and the ascending list of its set bits.

    Returns (ids int32 [count], count int, union words uint64 [f/64]).
    """
    bits = unpack_mask(np.asarray(words).reshape(batch, -1), f)
    union = np.zeros(f, dtype=bool)
    for b in range(batch):
        union |= bits[b]
    ids = np.flatnonzero(union).astype(np.int32)
    return ids, int(ids.size), pack_mask(union[None, :])[0]


# ---------------------------------------------------------------------------
# weights
# ---------------------------------------------------------------------------

def dequant_int4(q, s) -> np.ndarray:
    """[ciyun] 2.2: weight-only INT4 dequantised as w = q * s, exact in float64."""
    q = np.asarray(q, dtype=np.uint8)
    s = np.asarray(s, dtype=np.float16).astype(np.float64)
    rows, half = q.shape
    lo = (q & np.uint8(0x0F)).astype(np.int64)
    hi = (q >> np.uint8(4)).astype(np.int64)
    vals = np.empty((rows, 2 * half), dtype=np.int64)
    vals[:, 0::2] = lo
    vals[:, 1::2] = hi
    vals = np.where(vals >= 8, vals - 16, vals)
    scale = np.repeat(s, 128, axis=1)
    return vals.astype(np.float64) * scale


def rows_f64(layer, which: str, idx) -> np.ndarray:
    """Rows ``idx`` of W_up / W_gate / W_down^T in float64 (dequantised if INT4)."""
    idx = np.asarray(idx, dtype=np.int64)
    w = getattr(layer, "w_" + which)
    if w is not None:
        return np.asarray(w[idx], dtype=np.float64)
    q = getattr(layer, "q_" + which)
    s = getattr(layer, "s_" + which)
    return dequant_int4(q[idx], s[idx])


def _vec(v, n):
    return np.zeros(n, dtype=np.float64) if v is None else np.asarray(v, dtype=np.float64)


# ---------------------------------------------------------------------------
# the masked FFN  ([53ai] 激活稀疏: zero activations zero whole rows of the
# down projection, so those rows need neither loading nor multiplying)
# ---------------------------------------------------------------------------

def _phi(layer, rows_idx, xb):
    """phi_i(x) for the listed neurons: ReLU(up) or ReLU(gate) * up."""
    f = layer.spec.d_ff
    a = rows_f64(layer, "up", rows_idx) @ xb + _vec(layer.b_up, f)[rows_idx]
    if layer.spec.act == "relu":
        return np.maximum(a, 0.0)
    g = rows_f64(layer, "gate", rows_idx) @ xb + _vec(layer.b_gate, f)[rows_idx]
    return np.maximum(g, 0.0) * a


def masked_ffn(layer, x, bits, return_f64: bool = False):
    """y_b = b_down + sum over active i (ascending) of phi_i(x_b) * W_down[:, i].

    ``bits`` is the per-token mask [B][f] (bool) or packed words [B][f/64].
    Rows outside a token's mask are never read for that token.  The float64
    result is rounded once to float32.
    """
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    B = x.shape[0]
    d, f = layer.spec.d_model, layer.spec.d_ff
    m = np.asarray(bits)
    if m.dtype == np.uint64:
        m = unpack_mask(m.reshape(B, -1), f)
    m = np.atleast_2d(m).astype(bool)
    y = np.empty((B, d), dtype=np.float64)
    bd = _vec(layer.b_down, d)
    for b in range(B):
        ids = np.flatnonzero(m[b])
        acc = bd.copy()
        if ids.size:
            h = _phi(layer, ids, x[b])
            wd = rows_f64(layer, "down_t", ids)
            for k in range(ids.size):      # ascending neuron order
                acc += h[k] * wd[k]
        y[b] = acc
    return y if return_f64 else y.astype(np.float32)


def dense_ffn(layer, x, return_f64: bool = False):
    """The same FFN over every neuron: masked_ffn with an all-ones mask."""
    x = np.atleast_2d(np.asarray(x))
    ones = np.ones((x.shape[0], layer.spec.d_ff), dtype=bool)
    return masked_ffn(layer, x, ones, return_f64=return_f64)


def true_active(layer, x) -> np.ndarray:
    """[53ai] 验证上下文稀疏存在: the neurons whose output is non-zero.

    ReLU: up pre-activation > 0; ReGLU: gate pre-activation > 0 (and the
    product non-zero).  Returns [B][f] bool.
    """
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    f = layer.spec.d_ff
    allrows = np.arange(f)
    out = np.zeros((x.shape[0], f), dtype=bool)
    for b in range(x.shape[0]):
        out[b] = _phi(layer, allrows, x[b]) != 0.0
    return out


# ---------------------------------------------------------------------------
# offline profiling and hot-first layout  ([news] power-law paragraph;
# [53ai] 概述: the offline part separates hot from cold neurons)
# ---------------------------------------------------------------------------

def fire_counts(words, f: int) -> np.ndarray:
    """How often each neuron fires over a stack of masks [n][f/64] -> uint32 [f]."""
    bits = unpack_mask(np.asarray(words).reshape(-1, f // 64), f)
    return bits.sum(axis=0).astype(np.uint32)


def hot_first_perm(counts) -> np.ndarray:
    """Neuron order by descending fire count, ties by ascending index.

    perm[new_position] = original neuron id.
    """
    c = np.asarray(counts, dtype=np.int64)
    return np.lexsort((np.arange(c.size), -c)).astype(np.int32)


def permute_layer_ids(perm, ids_original):
    """Where original neurons land after the hot-first relayout (sorted)."""
    inv = np.empty_like(np.asarray(perm))
    inv[np.asarray(perm)] = np.arange(len(perm), dtype=inv.dtype)
    return np.sort(inv[np.asarray(ids_original, dtype=np.int64)]).astype(np.int32)


# ---------------------------------------------------------------------------
# stack driver step (pre-norm residual chain without gain)
# ---------------------------------------------------------------------------

def residual_rmsnorm(r, y, eps: float = 1e-6):
    """r' = r + y and x' = r' / sqrt(mean(r'^2) + eps), both float64."""
    r2 = np.atleast_2d(np.asarray(r, dtype=np.float64)) + np.atleast_2d(np.asarray(y, dtype=np.float64))
    ms = np.mean(r2 * r2, axis=1, keepdims=True)
    return r2, r2 / np.sqrt(ms + eps)


# ---------------------------------------------------------------------------
# input-sparse GEMV ([53ai] 第二阶段——插入新的ReLU)
# ---------------------------------------------------------------------------

def input_sparse_gemv(w_t, x, bias=None, return_f64: bool = False):
    """y = bias + W x for a batch of inputs with many zero entries, reading only
    the columns of W whose input is nonzero for some token of the batch.

    The relufication page's stage 2 puts a ReLU after the normalisation layer,
    so the inputs of the following projections (FFN up projection, attention
    QKV) are sparse and their zero entries select columns that contribute
    nothing.  W is stored input-major: w_t [n_in][n_out], row j is the column of
    W that input j multiplies.  J = the ascending indices j with x_b[j] != 0 for
    some token b (a -0.0 counts as zero, a NaN as nonzero); every token sums over
    J in ascending order:  y_b = bias + sum_{j in J} x_b[j] * w_t[j, :].
    A token's own zero entries in J add exact zeros, so y_b equals the dense
    product.  Returns (y [B][n_out] fp32, or fp64, and J as int64)."""
    x = np.asarray(x)
    w_t = np.asarray(w_t)
    J = np.flatnonzero(np.any(x != 0, axis=0))
    xb = x.astype(np.float64)
    y = np.zeros((x.shape[0], w_t.shape[1]), dtype=np.float64)
    if bias is not None:
        y += np.asarray(bias, dtype=np.float64)[None, :]
    for j in J:  # only the listed rows of w_t are read
        y += xb[:, j:j + 1] * w_t[j].astype(np.float64)[None, :]
    return (y if return_f64 else y.astype(np.float32)), J



# ---------------------------------------------------------------------------
# head-gated attention projections ([53ai] 如何充分利用结构化稀疏进行加速 and
# 验证上下文稀疏存在: only the heads predicted for an input are computed)
# ---------------------------------------------------------------------------

def head_qkv(w_qkv, b_qkv, x, head_bits, head_dim: int, return_f64: bool = False):
    """Q, K and V projections of the heads each token uses.

    w_qkv [3 H hd][d]: the q rows of head h are h*hd .. h*hd + hd - 1, then the
    k rows (offset H*hd) and the v rows (offset 2*H*hd).  out[t, r] is
    w_qkv[r] . x_t + b_qkv[r] when the head of row r is on for token t, else 0
    (a skipped head produces nothing).  head_bits [B][H] bool.
    """
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    w = np.asarray(w_qkv, dtype=np.float64)
    hb = np.atleast_2d(np.asarray(head_bits, dtype=bool))
    n = w.shape[0]
    H = n // (3 * head_dim)
    b = np.zeros(n) if b_qkv is None else np.asarray(b_qkv, dtype=np.float64)
    dense = x @ w.T + b[None, :]
    head_of_row = (np.arange(n) % (H * head_dim)) // head_dim
    out = np.where(hb[:, head_of_row], dense, 0.0)
    return out if return_f64 else out.astype(np.float32)


def head_out(w_o_t, b_o, attn, head_bits, head_dim: int, return_f64: bool = False):
    """Output projection over the heads each token uses.

    w_o_t [H hd][d] holds W_o's columns as rows (row j = column j); y_t =
    b_o + sum over heads h on for token t of attn_t[h hd : (h+1) hd] @ w_o_t
    [h hd : (h+1) hd].  Rows of heads that no token uses are never read.
    """
    a = np.atleast_2d(np.asarray(attn, dtype=np.float64))
    hb = np.atleast_2d(np.asarray(head_bits, dtype=bool))
    wt = np.asarray(w_o_t)
    B, n_in = a.shape
    d = wt.shape[1]
    H = n_in // head_dim
    y = np.zeros((B, d)) if b_o is None else np.tile(np.asarray(b_o, dtype=np.float64), (B, 1))
    for t in range(B):
        for h in range(H):
            if hb[t, h]:
                rows = slice(h * head_dim, (h + 1) * head_dim)
                y[t] += a[t, rows] @ wt[rows].astype(np.float64)
    return y if return_f64 else y.astype(np.float32)
