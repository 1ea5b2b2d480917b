"""Seeded synthetic layers and token streams shaped like the pages' models.

Sources for the shapes and statistics (all are used only as *shapes and
rates*; no trained weights or datasets exist here):

* 53ai.com sparsity survey, section "激活稀疏的可行性" (feasibility of activation
  sparsity): an OPT-6.7B ReLU FFN is more than 90% sparse.
* 53ai.com sparsity survey, section "性能对比" (performance comparison): about
  20% of OPT-30B's neurons fire per generated token.
* hexiedandong.com PowerInfer news page, power-law paragraph around figure (a):
  26% (OPT-30B) and 43% (LLaMA(ReGLU)-70B) of the neurons carry 80% of the
  activations.

Recipe (the plainest reading where the pages are silent):

* Weights N(0, 0.02), predictor factors N(0, 0.05), token vectors N(0, 1).
* Each neuron i has a fire probability p_i (uniform, or a clipped power law
  p_i = min(1, c * rank^-s) with (s, c) fitted so the top phi share of the sum
  of p is 0.80 and the mean is rho).  The rank -> neuron assignment is a
  seeded random permutation, so the natural layout is *not* hot-first.
* FFN bias b_i = -||w_i|| * Phi^-1(1 - p_i): for x ~ N(0, I) the
  pre-activation w_i.x + b_i is N(b_i, ||w_i||^2) and fires with probability
  p_i.  For ReGLU the calibrated bias goes on the gate row.
* Predictor threshold tau_i = sigma_i * Phi^-1(1 - p_i) with
  sigma_i = ||W1 W2[:, i]||, so the low-rank logit, which is N(0, sigma_i^2)
  for x ~ N(0, I), exceeds tau_i with probability p_i.
* INT4-g128: symmetric per (row, 128-group) scale s = fp16(max|w| / 7),
  q = clamp(round_half_even(w / s), -8, 7), two's complement nibbles with
  element 2k in the low nibble of byte k.

Every tensor is drawn from its own PCG64 stream keyed
SeedSequence(seed, spawn_key=(cfg, layer, tensor, chunk)) in fixed-size chunks,
so the bytes do not depend on how many threads draw them.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, field
from typing import Dict, Optional, Sequence

import numpy as np
from scipy.special import ndtri

_CHUNK = 1 << 22  # elements per independent RNG stream

# tensor ids inside a layer's key space
_T_WUP, _T_WGATE, _T_WDOWN, _T_W1, _T_W2, _T_PERM, _T_BDOWN = range(7)
_T_TOKENS = 100


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _stream(seed: int, key: Sequence[int]) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key))))


def _normal(shape, std: float, dtype, seed: int, key: Sequence[int]) -> np.ndarray:
    """N(0, std^2) drawn in fp32, scaled, cast once to ``dtype``."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=dtype)
    nchunk = (n + _CHUNK - 1) // _CHUNK

    def fill(c):
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        g = _stream(seed, tuple(key) + (c,))
        v = g.standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        out[lo:hi] = v.astype(dtype, copy=False)

    if nchunk == 1:
        fill(0)
    else:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunk)))
    return out.reshape(shape)


# ---------------------------------------------------------------------------
# fire-probability profiles
# ---------------------------------------------------------------------------

def uniform_probs(n: int, p: float) -> np.ndarray:
    return np.full(n, float(p), dtype=np.float64)


def _zipf_curve(n: int, s: float, c: float) -> np.ndarray:
    return np.minimum(1.0, c * np.arange(1, n + 1, dtype=np.float64) ** (-s))


def zipf_probs(n: int, phi: float, rho: float, share: float = 0.80):
    """Clipped power law p_rank = min(1, c * rank^-s), sorted descending.

    (s, c) are found by nested bisection: for a given s, c is set so the mean
    is ``rho``; then s is moved until the top round(phi * n) ranks hold
    ``share`` of the total.  Returns (p_by_rank, s, c).
    """
    k = int(round(phi * n))
    target = rho * n

    def c_for(s):
        # bisection on log c: the clipped mean is monotone in c
        lo, hi = -60.0, 60.0
        if _zipf_curve(n, s, np.exp(hi)).sum() < target:
            raise ValueError("rho unreachable")
        for _ in range(200):
            mid = 0.5 * (lo + hi)
            if _zipf_curve(n, s, np.exp(mid)).sum() < target:
                lo = mid
            else:
                hi = mid
        return float(np.exp(0.5 * (lo + hi)))

    def top_share(s):
        p = _zipf_curve(n, s, c_for(s))
        return p[:k].sum() / p.sum()

    s_lo, s_hi = 0.0, 4.0
    for _ in range(60):
        mid = 0.5 * (s_lo + s_hi)
        if top_share(mid) < share:
            s_lo = mid
        else:
            s_hi = mid
    s = 0.5 * (s_lo + s_hi)
    c = c_for(s)
    return _zipf_curve(n, s, c), s, c


def union_density(p: np.ndarray, batch: int) -> float:
    """Expected |U| / d_ff for ``batch`` i.i.d. tokens: mean_i 1 - (1 - p_i)^B."""
    p = np.asarray(p, dtype=np.float64)
    return float(np.mean(1.0 - (1.0 - p) ** batch))


# ---------------------------------------------------------------------------
# layer specs and the five workloads
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class LayerSpec:
    name: str
    cfg_id: int
    d_model: int
    d_ff: int
    rank: int
    wtype: str            # 'f32' | 'f16' | 'i4g128' (FFN weights)
    act: str              # 'relu' | 'reglu'
    pred_dtype: str       # 'f32' | 'f16'
    n_layers: int
    profile: str          # 'uniform' | 'zipf'
    rho: float            # mean fire probability
    phi: float = 0.0      # zipf: share of neurons holding 80% of the activations
    batches: tuple = (1,)
    w_std: float = 0.02
    p_std: float = 0.05
    has_b_up: bool = True

    @property
    def x_dtype(self):
        return np.float32 if self.wtype == "f32" else np.float16

    @property
    def n_mat(self) -> int:
        return 3 if self.act == "reglu" else 2


CONFIGS: Dict[str, LayerSpec] = {
    # OPT-125m-shaped single ReLU layer, fp32, rank-128 predictor, p = 0.1.
    "c1": LayerSpec("opt125m", 1, 768, 3072, 128, "f32", "relu", "f32", 1, "uniform", 0.10),
    # OPT-6.7B-shaped stack, fp16, rank-1024 predictor, ~90% sparse.
    "c2": LayerSpec("opt6.7b", 2, 4096, 16384, 1024, "f16", "relu", "f16", 32, "uniform", 0.10),
    # OPT-30B-shaped stack, power law: 26% of neurons carry 80%; ~20% active per token.
    "c3": LayerSpec("opt30b", 3, 7168, 28672, 1024, "f16", "relu", "f16", 48, "zipf", 0.20,
                    phi=0.26, batches=(1, 4, 16)),
    # LLaMA-ReGLU-70B-shaped gated FFN: 43% carry 80%; no biases except the calibrated gate bias.
    "c4": LayerSpec("llama-reglu70b", 4, 8192, 28672, 1024, "f16", "reglu", "f16", 80, "zipf", 0.10,
                    phi=0.43, batches=(1, 8), has_b_up=False),
    # OPT-175B-shaped INT4-g128 FFN, fp16 rank-1024 predictor, sparsity swept 85..95%.
    "c5": LayerSpec("opt175b-int4", 5, 12288, 49152, 1024, "i4g128", "relu", "f16", 96, "uniform", 0.10,
                    batches=(1, 2, 4, 32)),
}


def config(name: str, **overrides) -> LayerSpec:
    spec = CONFIGS[name]
    if overrides:
        d = dict(spec.__dict__)
        d.update(overrides)
        spec = LayerSpec(**d)
    return spec


@dataclass
class Layer:
    """One layer's tensors in storage layout (host numpy arrays).

    Neuron-major FFN: w_up, w_gate, w_down_t are [d_ff][d_model] (w_down_t row i
    is column i of the conventional W_down [d_model][d_ff]).  Predictor:
    w1_t [rank][d_model], w2_t [d_ff][rank], tau [d_ff] fp32.  INT4 layers keep
    the packed nibbles in q_* [d_ff][d_model/2] uint8 and scales s_* fp16
    [d_ff][d_model/128]; their w_* fields are None.
    """
    spec: LayerSpec
    probs: np.ndarray
    w1_t: np.ndarray
    w2_t: np.ndarray
    tau: np.ndarray
    w_up: Optional[np.ndarray] = None
    w_gate: Optional[np.ndarray] = None
    w_down_t: Optional[np.ndarray] = None
    q_up: Optional[np.ndarray] = None
    q_gate: Optional[np.ndarray] = None
    q_down_t: Optional[np.ndarray] = None
    s_up: Optional[np.ndarray] = None
    s_gate: Optional[np.ndarray] = None
    s_down_t: Optional[np.ndarray] = None
    b_up: Optional[np.ndarray] = None
    b_gate: Optional[np.ndarray] = None
    b_down: Optional[np.ndarray] = None
    extra: dict = field(default_factory=dict)

    def nbytes(self) -> int:
        return sum(v.nbytes for v in self.__dict__.values() if isinstance(v, np.ndarray))


def _probs_for(spec: LayerSpec, seed: int, layer: int) -> np.ndarray:
    n = spec.d_ff
    if spec.profile == "uniform":
        return uniform_probs(n, spec.rho)
    p_rank, _, _ = zipf_probs(n, spec.phi, spec.rho)
    perm = _stream(seed, (spec.cfg_id, layer, _T_PERM)).permutation(n)
    p = np.empty(n, dtype=np.float64)
    p[perm] = p_rank  # neuron perm[r] gets the r-th largest probability
    return p


def layer_probs(spec: LayerSpec, layer: int = 0, seed: int = 0) -> np.ndarray:
    """The per-neuron fire probabilities make_layer draws layer ``layer`` with."""
    return _probs_for(spec, seed, layer)


def _bias_for(norms: np.ndarray, p: np.ndarray) -> np.ndarray:
    """-||w|| Phi^-1(1-p); p = 1 -> +6||w|| (always on), p = 0 -> -6||w||."""
    pc = np.clip(p, 0.0, 1.0)
    z = np.where(pc >= 1.0, -6.0, np.where(pc <= 0.0, 6.0, ndtri(np.clip(1.0 - pc, 1e-300, 1.0))))
    z = np.clip(z, -6.0, 6.0)
    return -norms * z


def _row_norms(w: np.ndarray) -> np.ndarray:
    out = np.empty(w.shape[0], dtype=np.float64)

    def block(lo, hi):
        blk = w[lo:hi].astype(np.float64)
        out[lo:hi] = np.sqrt(np.einsum("ij,ij->i", blk, blk))

    _map_blocks(block, w.shape[0], 256)
    return out


def _tau_for(w1_t: np.ndarray, w2_t: np.ndarray, p: np.ndarray) -> np.ndarray:
    """sigma_i Phi^-1(1 - p_i) with sigma_i^2 = w2_t[i] G w2_t[i]^T, G = w1_t w1_t^T."""
    a = w1_t.astype(np.float64)
    g = a @ a.T
    sig2 = np.empty(w2_t.shape[0], dtype=np.float64)
    step = 4096
    for i in range(0, w2_t.shape[0], step):
        blk = w2_t[i:i + step].astype(np.float64)
        sig2[i:i + step] = np.einsum("ij,ij->i", blk @ g, blk)
    sigma = np.sqrt(np.maximum(sig2, 0.0))
    z = -_bias_for(np.ones_like(sigma), p)  # Phi^-1(1-p) with the same clipping
    return (sigma * z).astype(np.float32)


def _row_blocks(rows: int, step: int):
    return [(i, min(rows, i + step)) for i in range(0, rows, step)]


def _map_blocks(fn, rows: int, step: int):
    """Apply fn(lo, hi) to row blocks on a thread pool (NumPy releases the GIL
    inside its array loops); each block writes only its own rows."""
    blocks = _row_blocks(rows, step)
    if len(blocks) == 1:
        fn(*blocks[0])
        return
    with _cf.ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(lambda b: fn(*b), blocks))


def quant_int4_g128(w: np.ndarray):
    """Symmetric INT4, one fp16 scale per (row, 128 consecutive elements).

    Returns (q_packed uint8 [rows][cols/2], s fp16 [rows][cols/128]).
    Element 2k sits in the low nibble of byte k, two's complement.  Rows are
    independent, so row blocks are quantised in parallel.
    """
    rows, cols = w.shape
    assert cols % 128 == 0
    packed = np.empty((rows, cols // 2), dtype=np.uint8)
    s_out = np.empty((rows, cols // 128), dtype=np.float16)

    def block(lo, hi):
        wf = w[lo:hi].astype(np.float32).reshape(hi - lo, cols // 128, 128)
        amax = np.abs(wf).max(axis=2)
        s16 = (amax / np.float32(7.0)).astype(np.float16)
        s16 = np.where((s16 == 0) | ~np.isfinite(s16), np.float16(1.0), s16)
        sf = s16.astype(np.float32)[:, :, None]
        q = np.clip(np.rint(wf / sf), -8, 7).astype(np.int8).reshape(hi - lo, cols)
        u = (q.astype(np.int16) & 0xF).astype(np.uint8)
        packed[lo:hi] = u[:, 0::2] | (u[:, 1::2] << 4)
        s_out[lo:hi] = s16

    _map_blocks(block, rows, 1024)
    return packed, s_out


def _deq_norms_int4(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Row norms of the dequantised INT4 weights (used only to place biases)."""
    rows = q.shape[0]
    out = np.empty(rows, dtype=np.float64)

    def block(lo, hi):
        qb = q[lo:hi]
        low = (qb & 0xF).astype(np.int16)
        high = (qb >> 4).astype(np.int16)
        low = np.where(low >= 8, low - 16, low)
        high = np.where(high >= 8, high - 16, high)
        v = np.empty((qb.shape[0], qb.shape[1] * 2), dtype=np.float64)
        v[:, 0::2] = low
        v[:, 1::2] = high
        v *= np.repeat(s[lo:hi].astype(np.float64), 128, axis=1)
        out[lo:hi] = np.sqrt(np.einsum("ij,ij->i", v, v))

    _map_blocks(block, rows, 128)
    return out


def make_layer(spec: LayerSpec, layer: int = 0, seed: int = 0, probs: Optional[np.ndarray] = None,
               predictor: bool = True) -> Layer:
    """Draw one layer of ``spec`` (host arrays, storage dtypes)."""
    d, f, r = spec.d_model, spec.d_ff, spec.rank
    key = (spec.cfg_id, layer)
    p = _probs_for(spec, seed, layer) if probs is None else np.asarray(probs, dtype=np.float64)
    xdt = spec.x_dtype
    pdt = np.float32 if spec.pred_dtype == "f32" else np.float16
    wdt = np.float32 if spec.wtype == "f32" else np.float16

    lay = Layer(spec=spec, probs=p, w1_t=None, w2_t=None, tau=None)
    w_up = _normal((f, d), spec.w_std, wdt if spec.wtype != "i4g128" else np.float32, seed, key + (_T_WUP,))
    w_down = _normal((f, d), spec.w_std, wdt if spec.wtype != "i4g128" else np.float32, seed, key + (_T_WDOWN,))
    w_gate = None
    if spec.act == "reglu":
        w_gate = _normal((f, d), spec.w_std, wdt if spec.wtype != "i4g128" else np.float32, seed,
                         key + (_T_WGATE,))

    if spec.wtype == "i4g128":
        lay.q_up, lay.s_up = quant_int4_g128(w_up)
        lay.q_down_t, lay.s_down_t = quant_int4_g128(w_down)
        del w_up, w_down
        if w_gate is not None:
            lay.q_gate, lay.s_gate = quant_int4_g128(w_gate)
            del w_gate
        gate_norm = _deq_norms_int4(lay.q_gate, lay.s_gate) if spec.act == "reglu" else None
        up_norm = _deq_norms_int4(lay.q_up, lay.s_up) if spec.act == "relu" else None
    else:
        lay.w_up, lay.w_down_t, lay.w_gate = w_up, w_down, w_gate
        gate_norm = _row_norms(w_gate) if spec.act == "reglu" else None
        up_norm = _row_norms(w_up) if spec.act == "relu" else None

    if spec.act == "relu":
        lay.b_up = _bias_for(up_norm, p).astype(xdt)
    else:
        lay.b_gate = _bias_for(gate_norm, p).astype(xdt)
        lay.b_up = np.zeros(f, dtype=xdt) if spec.has_b_up else None
    lay.b_down = np.zeros(d, dtype=xdt)

    if predictor:
        lay.w1_t = _normal((r, d), spec.p_std, pdt, seed, key + (_T_W1,))
        lay.w2_t = _normal((f, r), spec.p_std, pdt, seed, key + (_T_W2,))
        lay.tau = _tau_for(lay.w1_t, lay.w2_t, p)
    return lay


def make_tokens(spec: LayerSpec, n: int, seed: int = 0, stream: int = 0, dtype=None) -> np.ndarray:
    """n token vectors x ~ N(0, I) of length d_model, [n][d] in x dtype (or ``dtype``)."""
    dt = spec.x_dtype if dtype is None else dtype
    return _normal((n, spec.d_model), 1.0, dt, seed, (spec.cfg_id, _T_TOKENS, stream))


# ---------------------------------------------------------------------------
# integer-grid fixtures (every intermediate is an integer below 2^24)
# ---------------------------------------------------------------------------

def make_grid_layer(d: int, f: int, r: int, act: str = "relu", wtype: str = "f16", seed: int = 0,
                    tensor_scale: int = 0) -> Layer:
    """Weights, x-compatible biases and predictor factors in {-2..2} (times 2^tensor_scale).

    Biases are integers in [-8, 8]; tau are half-integers so no logit ties.
    For INT4 the nibbles are drawn in [-2, 2] with power-of-two scales.
    """
    g = _stream(seed, (9, d, f, r, 0 if act == "relu" else 1))
    sc = float(2.0 ** tensor_scale)
    xdt = np.float32 if wtype == "f32" else np.float16
    wdt = np.float32 if wtype == "f32" else np.float16
    spec = LayerSpec(f"grid{d}x{f}", 9, d, f, r, wtype, act, "f32" if wtype == "f32" else "f16", 1,
                     "uniform", 0.5)

    def ints(shape, lo, hi):
        return g.integers(lo, hi + 1, size=shape).astype(np.float64)

    lay = Layer(spec=spec, probs=np.full(f, 0.5), w1_t=None, w2_t=None, tau=None)
    if wtype == "i4g128":
        def q4(shape):
            qv = g.integers(-2, 3, size=shape).astype(np.int16)
            u = (qv & 0xF).astype(np.uint8)
            return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)

        def s4(shape):
            return (2.0 ** g.integers(-1, 2, size=shape)).astype(np.float16)

        lay.q_up, lay.s_up = q4((f, d)), s4((f, d // 128))
        lay.q_down_t, lay.s_down_t = q4((f, d)), s4((f, d // 128))
        if act == "reglu":
            lay.q_gate, lay.s_gate = q4((f, d)), s4((f, d // 128))
    else:
        lay.w_up = (ints((f, d), -2, 2) * sc).astype(wdt)
        lay.w_down_t = (ints((f, d), -2, 2)).astype(wdt)
        if act == "reglu":
            lay.w_gate = (ints((f, d), -2, 2) * sc).astype(wdt)
    lay.b_up = (ints((f,), -8, 8) * sc).astype(xdt)
    if act == "reglu":
        lay.b_gate = (ints((f,), -8, 8) * sc).astype(xdt)
    lay.b_down = ints((d,), -4, 4).astype(xdt)
    pdt = np.float32 if wtype == "f32" else np.float16
    lay.w1_t = ints((r, d), -2, 2).astype(pdt)
    lay.w2_t = ints((f, r), -2, 2).astype(pdt)
    lay.tau = (ints((f,), -40, 40) + 0.5).astype(np.float32)
    return lay


def make_grid_tokens(d: int, n: int, seed: int = 0, dtype=np.float16) -> np.ndarray:
    g = _stream(seed, (10, d, n))
    return g.integers(-2, 3, size=(n, d)).astype(dtype)


# ---------------------------------------------------------------------------
# mask inputs for compaction tests
# ---------------------------------------------------------------------------

def pack_bits(bits: np.ndarray) -> np.ndarray:
    """[..., f] bool -> [..., f/64] uint64, bit i%64 of word i/64 (LSB first)."""
    bits = np.asarray(bits, dtype=bool)
    f = bits.shape[-1]
    assert f % 64 == 0
    b = bits.reshape(bits.shape[:-1] + (f // 64, 64)).astype(np.uint64)
    w = np.zeros(b.shape[:-1], dtype=np.uint64)
    for j in range(64):
        w |= b[..., j] << np.uint64(j)
    return w


def random_masks(batch: int, f: int, density: float, seed: int = 0, probs=None) -> np.ndarray:
    """Packed [batch][f/64] masks with i.i.d. bits of the given density (or per-neuron probs)."""
    g = _stream(seed, (11, batch, f, int(density * 1e6)))
    p = np.full(f, density) if probs is None else np.asarray(probs)
    bits = g.random((batch, f)) < p[None, :]
    return pack_bits(bits)


# ---------------------------------------------------------------------------
# input-sparse GEMV inputs (relufication stage 2: a ReLU inserted after the
# normalisation layer, [53ai] 第二阶段——插入新的ReLU)
# ---------------------------------------------------------------------------

_T_ISG_W, _T_ISG_B, _T_ISG_X = 200, 201, 202


def make_isg_weights(n_in: int, n_out: int, wtype: str = "f16", seed: int = 0, key: int = 0,
                     bias: bool = True):
    """A projection stored input-major: w_t [n_in][n_out] ~ N(0, 0.02^2) (row j is
    the column of W that input j multiplies), and a bias [n_out] ~ N(0, 0.02^2)
    (or None).  Storage dtype fp16 or fp32."""
    dt = np.float32 if wtype == "f32" else np.float16
    w_t = _normal((n_in, n_out), 0.02, dt, seed, (_T_ISG_W, key))
    b = _normal((n_out,), 0.02, dt, seed, (_T_ISG_B, key)) if bias else None
    return w_t, b


def make_relu_inputs(n_in: int, n: int, density: float, seed: int = 0, stream: int = 0,
                     dtype=np.float16) -> np.ndarray:
    """n input vectors as a ReLU after a normalisation layer would hand them on:
    x = max(z - theta, 0) with z ~ N(0, 1) and theta = Phi^-1(1 - density), so
    each entry is nonzero with probability ``density`` (theta = 0 at 0.5, the
    plain ReLU of a normalised input)."""
    theta = 0.0 if density >= 1.0 else float(ndtri(1.0 - density)) if density > 0.0 else np.inf
    z = _stream(seed, (_T_ISG_X, n_in, n, stream)).standard_normal((n, n_in), dtype=np.float32)
    if density >= 1.0:
        x = z  # every entry kept: the dense input
    else:
        x = np.maximum(z - np.float32(theta), np.float32(0.0))
    return x.astype(dtype)



# ---- head-gated attention projections ----------------------------------------

_T_HEAD_W, _T_HEAD_B, _T_HEAD_M = 210, 211, 212


def make_head_weights(d: int, n_heads: int, head_dim: int, wtype: str = "f16", seed: int = 0,
                      bias: bool = True):
    """One attention block's projections in storage layout, N(0, 0.02^2):
    w_qkv [3 H hd][d] (q rows of all heads, then k, then v), b_qkv [3 H hd],
    w_o_t [H hd][d] (row j is column j of W_o), b_o [d] (biases None when
    ``bias`` is False).  Storage dtype fp16 or fp32."""
    dt = np.float32 if wtype == "f32" else np.float16
    n = n_heads * head_dim
    w_qkv = _normal((3 * n, d), 0.02, dt, seed, (_T_HEAD_W, 0))
    w_o_t = _normal((n, d), 0.02, dt, seed, (_T_HEAD_W, 1))
    b_qkv = _normal((3 * n,), 0.02, dt, seed, (_T_HEAD_B, 0)) if bias else None
    b_o = _normal((d,), 0.02, dt, seed, (_T_HEAD_B, 1)) if bias else None
    return w_qkv, b_qkv, w_o_t, b_o


def make_head_masks(batch: int, n_heads: int, density: float, seed: int = 0):
    """Per-token head sets: each head on with probability ``density`` (the
    pages report up to 80% of heads skipped, i.e. density 0.2).  Returns the
    bits [B][H] and the packed words [B][ceil(H/64)]."""
    g = _stream(seed, (_T_HEAD_M, batch, n_heads))
    bits = g.random((batch, n_heads)) < density
    pad = np.zeros((batch, (n_heads + 63) // 64 * 64), dtype=bool)
    pad[:, :n_heads] = bits
    return bits, pack_bits(pad)
