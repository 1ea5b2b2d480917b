"""ctypes binding of libsfnn.so: the C entry points under the same names.

Argument marshalling only.  Every computation runs in the HIP kernels of
libsfnn.so; if the library is missing this module raises instead of falling
back to anything else.  torch is imported first so the library binds to the
HIP runtime torch already loaded (tensors give device pointers, the current
torch stream gives the hipStream_t).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsfnn.so")

SFNN_F32, SFNN_F16, SFNN_I4G128 = 0, 1, 2
SFNN_RELU, SFNN_REGLU = 0, 1
STATUS = {0: "SFNN_OK", 1: "SFNN_E_NULL", 2: "SFNN_E_SHAPE", 3: "SFNN_E_ALIGN", 4: "SFNN_E_DTYPE",
          5: "SFNN_E_WORKSPACE", 6: "SFNN_E_HIP"}

EXPORTS = [
    "sfnn_workspace_bytes", "sfnn_predict", "sfnn_compact", "sfnn_sparse_ffn", "sfnn_dense_ffn",
    "sfnn_layer", "sfnn_stack_decode", "sfnn_residual_rmsnorm", "sfnn_fire_counts", "sfnn_hot_first_perm",
    "sfnn_gather_rows", "sfnn_probe_read", "sfnn_probe_copy", "sfnn_status_str", "sfnn_version",
    "sfnn_isg_workspace_bytes", "sfnn_input_sparse_gemv", "sfnn_heads_workspace_bytes", "sfnn_head_qkv",
    "sfnn_head_out", "sfnn_layer_noalloc", "sfnn_dense_min_batch",
]


class SfnnError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} returned {STATUS.get(code, code)}")
        self.code = code


class sfnn_pred(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("wtype", ctypes.c_int32), ("w1_t", ctypes.c_void_p), ("w2_t", ctypes.c_void_p),
                ("tau", ctypes.c_void_p), ("hot_prefix", ctypes.c_int32), ("dense_min_batch", ctypes.c_int32)]


class sfnn_ffn(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("wtype", ctypes.c_int32),
                ("act", ctypes.c_int32),
                ("w_up", ctypes.c_void_p), ("w_gate", ctypes.c_void_p), ("w_down_t", ctypes.c_void_p),
                ("s_up", ctypes.c_void_p), ("s_gate", ctypes.c_void_p), ("s_down_t", ctypes.c_void_p),
                ("b_up", ctypes.c_void_p), ("b_gate", ctypes.c_void_p), ("b_down", ctypes.c_void_p),
                ("mfma_min_batch", ctypes.c_int32)]


class sfnn_isg(ctypes.Structure):
    _fields_ = [("n_in", ctypes.c_int32), ("n_out", ctypes.c_int32), ("wtype", ctypes.c_int32),
                ("w_t", ctypes.c_void_p), ("bias", ctypes.c_void_p)]


class sfnn_heads(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("wtype", ctypes.c_int32), ("w_qkv", ctypes.c_void_p), ("b_qkv", ctypes.c_void_p),
                ("w_o_t", ctypes.c_void_p), ("b_o", ctypes.c_void_p)]


_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libsfnn.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m activation_sparse_gemv_amd.build`")
    L = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    P, F, G = ctypes.POINTER(sfnn_pred), ctypes.POINTER(sfnn_ffn), ctypes.POINTER(sfnn_isg)
    Hd = ctypes.POINTER(sfnn_heads)
    sig = {
        "sfnn_workspace_bytes": (sz, [P, F, i32]),
        "sfnn_predict": (i32, [P, vp, i32, vp, vp, vp, sz, vp]),
        "sfnn_compact": (i32, [vp, i32, i32, vp, vp, vp, vp]),
        "sfnn_sparse_ffn": (i32, [F, vp, i32, vp, vp, vp, vp, vp, sz, vp]),
        "sfnn_dense_ffn": (i32, [F, vp, i32, vp, vp, sz, vp]),
        "sfnn_layer": (i32, [P, F, vp, i32, vp, vp, vp, vp, vp, sz, vp]),
        "sfnn_layer_noalloc": (i32, [P, F, vp, i32, vp, vp, vp, vp, vp]),
        "sfnn_stack_decode": (i32, [i32, P, F, i32, vp, vp, ctypes.c_float, i32, vp, vp, vp, vp, vp, vp, sz, vp]),
        "sfnn_residual_rmsnorm": (i32, [vp, vp, vp, i32, i32, ctypes.c_float, vp, i32, vp]),
        "sfnn_fire_counts": (i32, [vp, i32, i32, vp, vp]),
        "sfnn_hot_first_perm": (i32, [vp, i32, vp]),
        "sfnn_dense_min_batch": (i32, [vp, i32, i32, ctypes.c_float, i32, vp]),
        "sfnn_gather_rows": (i32, [vp, vp, i32, i64, vp, vp]),
        "sfnn_probe_read": (i32, [vp, sz, vp, vp]),
        "sfnn_probe_copy": (i32, [vp, vp, sz, vp]),
        "sfnn_status_str": (ctypes.c_char_p, [i32]),
        "sfnn_isg_workspace_bytes": (sz, [G, i32]),
        "sfnn_input_sparse_gemv": (i32, [G, vp, i32, vp, vp, vp, vp, sz, vp]),
        "sfnn_heads_workspace_bytes": (sz, [Hd, i32]),
        "sfnn_head_qkv": (i32, [Hd, vp, i32, vp, vp, vp]),
        "sfnn_head_out": (i32, [Hd, vp, i32, vp, vp, vp, sz, vp]),
        "sfnn_version": (i32, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _p(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _s(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, code: int):
    if code != 0:
        raise SfnnError(fn, code)


def _wtype_of(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SFNN_F32
    if t.dtype == torch.float16:
        return SFNN_F16
    if t.dtype == torch.uint8:
        return SFNN_I4G128
    raise TypeError(f"unsupported weight dtype {t.dtype}")


class Pred:
    """Device predictor descriptor (keeps its tensors alive)."""

    def __init__(self, w1_t: torch.Tensor, w2_t: torch.Tensor, tau: torch.Tensor, hot_prefix: int = 0,
                 dense_min_batch: int = 0):
        self.w1_t, self.w2_t, self.tau = w1_t, w2_t, tau
        r, d = w1_t.shape
        f = w2_t.shape[0]
        self.c = sfnn_pred(d, f, r, _wtype_of(w1_t), _p(w1_t), _p(w2_t), _p(tau), hot_prefix, dense_min_batch)

    @property
    def hot_prefix(self) -> int:
        return self.c.hot_prefix

    @hot_prefix.setter
    def hot_prefix(self, h: int):
        self.c.hot_prefix = h

    @property
    def dense_min_batch(self) -> int:
        """Batch from which sfnn_layer / sfnn_stack_decode run dense (<= 0: never)."""
        return self.c.dense_min_batch

    @dense_min_batch.setter
    def dense_min_batch(self, b: int):
        self.c.dense_min_batch = b

    @property
    def ref(self):
        return ctypes.byref(self.c)


class FFN:
    """Device FFN descriptor (keeps its tensors alive)."""

    def __init__(self, w_up, w_down_t, act: int = SFNN_RELU, w_gate=None, s_up=None, s_gate=None,
                 s_down_t=None, b_up=None, b_gate=None, b_down=None, mfma_min_batch: int = 0):
        self.t = dict(w_up=w_up, w_gate=w_gate, w_down_t=w_down_t, s_up=s_up, s_gate=s_gate,
                      s_down_t=s_down_t, b_up=b_up, b_gate=b_gate, b_down=b_down)
        wt = _wtype_of(w_up)
        f = w_up.shape[0]
        d = w_up.shape[1] * (2 if wt == SFNN_I4G128 else 1)
        self.d_model, self.d_ff, self.wtype, self.act = d, f, wt, act
        self.c = sfnn_ffn(d, f, wt, act, *[_p(self.t[k]) for k in
                                           ("w_up", "w_gate", "w_down_t", "s_up", "s_gate", "s_down_t",
                                            "b_up", "b_gate", "b_down")], mfma_min_batch)

    @property
    def mfma_min_batch(self) -> int:
        """Batch size from which an fp16 FFN runs on the matrix cores (0: the
        library default, negative: never); read by every call."""
        return int(self.c.mfma_min_batch)

    @mfma_min_batch.setter
    def mfma_min_batch(self, v: int):
        self.c.mfma_min_batch = int(v)

    @property
    def ref(self):
        return ctypes.byref(self.c)


class Isg:
    """Device descriptor of an input-sparse GEMV (keeps its tensors alive):
    w_t [n_in][n_out] fp16 or fp32, bias [n_out] or None."""

    def __init__(self, w_t: torch.Tensor, bias: Optional[torch.Tensor] = None):
        self.w_t, self.bias = w_t, bias
        self.n_in, self.n_out = w_t.shape
        self.c = sfnn_isg(self.n_in, self.n_out, _wtype_of(w_t), _p(w_t), _p(bias))

    @property
    def ref(self):
        return ctypes.byref(self.c)


def _ref(desc):
    return None if desc is None else desc.ref


# ---------------------------------------------------------------------------
# the C entry points, same names
# ---------------------------------------------------------------------------

def sfnn_workspace_bytes(pred: Optional[Pred], ffn: Optional[FFN], batch: int) -> int:
    return int(load().sfnn_workspace_bytes(_ref(pred), _ref(ffn), batch))


def sfnn_predict(pred: Pred, x, batch: int, mask, logits, ws, stream=None):
    _check("sfnn_predict", load().sfnn_predict(pred.ref, _p(x), batch, _p(mask), _p(logits), _p(ws),
                                                ws.numel() * ws.element_size(), _s(stream)))


def sfnn_compact(mask, batch: int, d_ff: int, ids, count, union_mask=None, stream=None):
    _check("sfnn_compact", load().sfnn_compact(_p(mask), batch, d_ff, _p(ids), _p(count), _p(union_mask),
                                                _s(stream)))


def sfnn_sparse_ffn(ffn: FFN, x, batch: int, ids, count, mask, y, ws, stream=None):
    _check("sfnn_sparse_ffn", load().sfnn_sparse_ffn(ffn.ref, _p(x), batch, _p(ids), _p(count), _p(mask), _p(y),
                                                      _p(ws), ws.numel() * ws.element_size(), _s(stream)))


def sfnn_dense_ffn(ffn: FFN, x, batch: int, y, ws, stream=None):
    _check("sfnn_dense_ffn", load().sfnn_dense_ffn(ffn.ref, _p(x), batch, _p(y), _p(ws),
                                                    ws.numel() * ws.element_size(), _s(stream)))


def sfnn_layer(pred: Pred, ffn: FFN, x, batch: int, y, mask=None, ids=None, count=None, ws=None, stream=None):
    _check("sfnn_layer", load().sfnn_layer(pred.ref, ffn.ref, _p(x), batch, _p(y), _p(mask), _p(ids), _p(count),
                                            _p(ws), ws.numel() * ws.element_size(), _s(stream)))


SFNN_NOALLOC_SCRATCH_BYTES = 32 << 20  # the library's per-GPU scratch array (include/sfnn.h)


def sfnn_layer_noalloc(pred: Pred, ffn: FFN, x, batch: int, y, mask=None, ids=None, count=None, stream=None):
    _check("sfnn_layer_noalloc", load().sfnn_layer_noalloc(pred.ref, ffn.ref, _p(x), batch, _p(y), _p(mask), _p(ids),
                                                            _p(count), _s(stream)))


class Stack:
    """Host arrays of per-layer descriptors for sfnn_stack_decode (keeps the layers alive).
    The descriptors are copied here: a later change to a layer's Pred or FFN
    fields (hot_prefix, dense_min_batch, ...) needs a new Stack."""

    def __init__(self, layers):
        self.layers = list(layers)  # [(Pred, FFN)]
        n = len(self.layers)
        self.preds = (sfnn_pred * n)(*[p.c for p, _ in self.layers])
        self.ffns = (sfnn_ffn * n)(*[f.c for _, f in self.layers])

    def __len__(self):
        return len(self.layers)


SFNN_STACK_LOOKAHEAD = 1


def sfnn_stack_decode(stack: Stack, batch: int, r_in, r_out, eps: float, ws, flags: int = 0, x_cap=None, y_cap=None,
                      mask_cap=None, ids_cap=None, count_cap=None, stream=None):
    _check("sfnn_stack_decode", load().sfnn_stack_decode(
        len(stack), stack.preds, stack.ffns, batch, _p(r_in), _p(r_out), eps, flags, _p(x_cap), _p(y_cap),
        _p(mask_cap), _p(ids_cap), _p(count_cap), _p(ws), ws.numel() * ws.element_size(), _s(stream)))


def sfnn_residual_rmsnorm(r_in, y, r_out, batch: int, d_model: int, eps: float, x_out, stream=None):
    xt = SFNN_F32 if x_out.dtype == torch.float32 else SFNN_F16
    _check("sfnn_residual_rmsnorm", load().sfnn_residual_rmsnorm(_p(r_in), _p(y), _p(r_out), batch, d_model, eps,
                                                                  _p(x_out), xt, _s(stream)))


def sfnn_fire_counts(masks, n_masks: int, d_ff: int, counts, stream=None):
    _check("sfnn_fire_counts", load().sfnn_fire_counts(_p(masks), n_masks, d_ff, _p(counts), _s(stream)))


def sfnn_hot_first_perm(counts_host, d_ff: int, perm_host):
    """Host call: counts_host uint32 and perm_host int32 are CPU tensors or numpy arrays."""
    cp = counts_host.ctypes.data if hasattr(counts_host, "ctypes") else counts_host.data_ptr()
    pp = perm_host.ctypes.data if hasattr(perm_host, "ctypes") else perm_host.data_ptr()
    _check("sfnn_hot_first_perm", load().sfnn_hot_first_perm(cp, d_ff, pp))


def sfnn_dense_min_batch(counts_host, n_profiled: int, d_ff: int, crossover: float, max_batch: int) -> int:
    """Host call: the dense-switch threshold for fire counts (uint32 CPU tensor
    or numpy array) over n_profiled tokens; -1 when no batch up to max_batch
    reaches the crossover share."""
    cp = counts_host.ctypes.data if hasattr(counts_host, "ctypes") else counts_host.data_ptr()
    out = ctypes.c_int32(0)
    _check("sfnn_dense_min_batch",
           load().sfnn_dense_min_batch(cp, n_profiled, d_ff, float(crossover), max_batch, ctypes.byref(out)))
    return out.value


def sfnn_gather_rows(src, perm, n_rows: int, row_bytes: int, dst, stream=None):
    _check("sfnn_gather_rows", load().sfnn_gather_rows(_p(src), _p(perm), n_rows, row_bytes, _p(dst), _s(stream)))


def sfnn_probe_read(buf, nbytes: int, sink, stream=None):
    _check("sfnn_probe_read", load().sfnn_probe_read(_p(buf), nbytes, _p(sink), _s(stream)))


def sfnn_probe_copy(src, dst, nbytes: int, stream=None):
    _check("sfnn_probe_copy", load().sfnn_probe_copy(_p(src), _p(dst), nbytes, _s(stream)))


def sfnn_status_str(code: int) -> str:
    return load().sfnn_status_str(code).decode()


def sfnn_version() -> int:
    return int(load().sfnn_version())


class Heads:
    """Device descriptor of one attention block's projections (keeps its tensors
    alive): w_qkv [3 H hd][d], w_o_t [H hd][d] fp16 or fp32, biases or None."""

    def __init__(self, w_qkv: torch.Tensor, w_o_t: torch.Tensor, head_dim: int, b_qkv=None, b_o=None):
        self.t = dict(w_qkv=w_qkv, w_o_t=w_o_t, b_qkv=b_qkv, b_o=b_o)
        n, d = w_o_t.shape
        self.d_model, self.head_dim, self.n_heads = d, head_dim, n // head_dim
        self.c = sfnn_heads(d, self.n_heads, head_dim, _wtype_of(w_qkv), _p(w_qkv), _p(b_qkv), _p(w_o_t), _p(b_o))

    @property
    def ref(self):
        return ctypes.byref(self.c)


def sfnn_heads_workspace_bytes(op: Heads, batch: int) -> int:
    return int(load().sfnn_heads_workspace_bytes(op.ref, batch))


def sfnn_head_qkv(op: Heads, x, batch: int, head_mask, qkv, stream=None):
    _check("sfnn_head_qkv", load().sfnn_head_qkv(op.ref, _p(x), batch, _p(head_mask), _p(qkv), _s(stream)))


def sfnn_head_out(op: Heads, attn, batch: int, head_mask, y, ws, stream=None):
    _check("sfnn_head_out", load().sfnn_head_out(op.ref, _p(attn), batch, _p(head_mask), _p(y), _p(ws),
                                                 ws.numel() * ws.element_size(), _s(stream)))


def sfnn_isg_workspace_bytes(op: Isg, batch: int) -> int:
    return int(load().sfnn_isg_workspace_bytes(op.ref, batch))


def sfnn_input_sparse_gemv(op: Isg, x, batch: int, y, ws, cols=None, count=None, stream=None):
    _check("sfnn_input_sparse_gemv", load().sfnn_input_sparse_gemv(op.ref, _p(x), batch, _p(y), _p(cols), _p(count),
                                                                    _p(ws), ws.numel() * ws.element_size(),
                                                                    _s(stream)))

