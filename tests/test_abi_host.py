"""Host-side checks of the C-ABI library (no GPU needed): it loads, exports
every symbol the header declares, validates arguments before launching, and
the host-only helpers (hot-first ordering, dense-switch threshold) are right."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_symbols():
    txt = open(os.path.join(ROOT, "include", "sfnn.h")).read()
    return sorted(set(re.findall(r"\b(sfnn_[a-z_]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def L():
    import activation_sparse_gemv_amd as m
    return m.load()


def test_exports_match_header(L):
    import activation_sparse_gemv_amd as m
    syms = header_symbols()
    assert len(syms) >= 14
    assert sorted(m.EXPORTS) == syms
    for s in syms:
        assert hasattr(L, s), s


def test_version_and_status_strings(L):
    import activation_sparse_gemv_amd as m
    assert m.sfnn_version() >= 350  # 350: sfnn_dense_min_batch, per-layer stack switch
    assert m.sfnn_status_str(0) == "ok"
    assert "workspace" in m.sfnn_status_str(5)


def test_validation_rejects_without_launching(L):
    import activation_sparse_gemv_amd as m
    P = m._lib.sfnn_pred
    F = m._lib.sfnn_ffn
    fake = 1 << 20  # aligned non-null host value; never dereferenced because validation fails first
    # null descriptor
    assert L.sfnn_predict(None, fake, 1, fake, None, fake, 1 << 30, None) == 1
    # bad shapes
    p = P(768, 3000, 128, 0, fake, fake, fake)          # d_ff % 64 != 0
    assert L.sfnn_predict(ctypes.byref(p), fake, 1, fake, None, fake, 1 << 30, None) == 2
    p = P(768, 3072, 128, 0, fake, fake, fake)
    assert L.sfnn_predict(ctypes.byref(p), fake, 0, fake, None, fake, 1 << 30, None) == 2   # batch 0
    assert L.sfnn_predict(ctypes.byref(p), fake, 65, fake, None, fake, 1 << 30, None) == 2  # batch 65
    assert L.sfnn_predict(ctypes.byref(p), fake + 4, 1, fake, None, fake, 1 << 30, None) == 3  # misaligned
    assert L.sfnn_predict(ctypes.byref(p), fake, 1, fake, None, fake, 16, None) == 5          # workspace
    p.wtype = 2
    assert L.sfnn_predict(ctypes.byref(p), fake, 1, fake, None, fake, 1 << 30, None) == 4     # INT4 predictor
    for hot in (32, -64, 3072 + 64):  # dense hot prefix: a multiple of 64 within [0, d_ff]
        p = P(768, 3072, 128, 0, fake, fake, fake, hot)
        assert L.sfnn_predict(ctypes.byref(p), fake, 1, fake, None, fake, 1 << 30, None) == 2
        assert L.sfnn_workspace_bytes(ctypes.byref(p), None, 1) == 0
    p = P(768, 3072, 128, 0, fake, fake, fake, 3072)
    assert L.sfnn_workspace_bytes(ctypes.byref(p), None, 1) > 0
    f = F(768, 3072, 1, 1, fake, None, fake, None, None, None, None, None, None)         # ReGLU w/o gate
    assert L.sfnn_sparse_ffn(ctypes.byref(f), fake, 1, fake, fake, None, fake, fake, 1 << 30, None) == 1
    f = F(700, 3072, 1, 0, fake, None, fake, None, None, None, None, None, None)         # d_model % 128
    assert L.sfnn_sparse_ffn(ctypes.byref(f), fake, 1, fake, fake, None, fake, fake, 1 << 30, None) == 2
    f = F(768, 3072, 2, 0, fake, None, fake, None, None, None, None, None, None)         # INT4 w/o scales
    assert L.sfnn_dense_ffn(ctypes.byref(f), fake, 1, fake, fake, 1 << 30, None) == 1
    assert L.sfnn_compact(fake, 1, 100, fake, fake, None, None) == 2
    assert L.sfnn_compact(None, 1, 128, fake, fake, None, None) == 1
    # layer: predictor / ffn type mismatch
    p = P(768, 3072, 128, 1, fake, fake, fake)
    f = F(768, 3072, 0, 0, fake, None, fake, None, None, None, None, None, None)
    assert L.sfnn_layer(ctypes.byref(p), ctypes.byref(f), fake, 1, fake, None, None, None, fake, 1 << 30,
                        None) == 4


def test_workspace_bytes(L):
    import activation_sparse_gemv_amd as m
    P, F = m._lib.sfnn_pred, m._lib.sfnn_ffn
    fake = 1 << 20
    p = P(4096, 16384, 1024, 1, fake, fake, fake)
    f = F(4096, 16384, 1, 0, fake, None, fake, None, None, None, None, None, None)
    n1 = L.sfnn_workspace_bytes(ctypes.byref(p), ctypes.byref(f), 1)
    n8 = L.sfnn_workspace_bytes(ctypes.byref(p), ctypes.byref(f), 8)
    assert n1 >= 1024 * 4 + 16384 * 4 + 16384 * 4 and n8 > n1 and n1 % 256 == 0
    assert L.sfnn_workspace_bytes(ctypes.byref(p), ctypes.byref(f), 0) == 0
    assert L.sfnn_workspace_bytes(None, None, 1) == 0


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_hot_first_perm_host_matches_oracle(L, seed):
    import activation_sparse_gemv_amd as m
    g = np.random.default_rng(seed)
    f = 4096
    counts = g.integers(0, 20, size=f).astype(np.uint32)    # many ties
    perm = np.empty(f, dtype=np.int32)
    m.sfnn_hot_first_perm(counts, f, perm)
    assert np.array_equal(perm, oracle.hot_first_perm(counts))


def test_isg_validation_and_workspace(L):
    import activation_sparse_gemv_amd as m
    G = m._lib.sfnn_isg
    fake = 1 << 20
    ok = G(4096, 16384, 1, fake, None)
    ws = L.sfnn_isg_workspace_bytes(ctypes.byref(ok), 1)
    assert ws > 16384 * 4  # at least one partial row set
    assert L.sfnn_isg_workspace_bytes(ctypes.byref(ok), 2) > ws
    assert L.sfnn_isg_workspace_bytes(ctypes.byref(ok), 0) == 0
    assert L.sfnn_input_sparse_gemv(None, fake, 1, fake, None, None, fake, 1 << 30, None) == 1
    bad = G(4000, 16384, 1, fake, None)   # n_in % 64
    assert L.sfnn_isg_workspace_bytes(ctypes.byref(bad), 1) == 0
    assert L.sfnn_input_sparse_gemv(ctypes.byref(bad), fake, 1, fake, None, None, fake, 1 << 30, None) == 2
    bad = G(4096, 1000, 1, fake, None)    # n_out % 128
    assert L.sfnn_input_sparse_gemv(ctypes.byref(bad), fake, 1, fake, None, None, fake, 1 << 30, None) == 2
    bad = G(4096, 16384, 2, fake, None)   # INT4 is not an input-sparse GEMV type
    assert L.sfnn_input_sparse_gemv(ctypes.byref(bad), fake, 1, fake, None, None, fake, 1 << 30, None) == 4
    assert L.sfnn_input_sparse_gemv(ctypes.byref(ok), fake, 65, fake, None, None, fake, 1 << 30, None) == 2
    assert L.sfnn_input_sparse_gemv(ctypes.byref(ok), fake + 4, 1, fake, None, None, fake, 1 << 30, None) == 3
    assert L.sfnn_input_sparse_gemv(ctypes.byref(ok), fake, 1, fake, None, fake + 2, fake, 1 << 30, None) == 3
    assert L.sfnn_input_sparse_gemv(ctypes.byref(ok), fake, 1, fake, None, None, fake, 64, None) == 5


def test_heads_validation_and_workspace(L):
    import activation_sparse_gemv_amd as m
    H = m._lib.sfnn_heads
    fake = 1 << 20
    ok = H(4096, 32, 128, 1, fake, None, fake, None)
    ws = L.sfnn_heads_workspace_bytes(ctypes.byref(ok), 1)
    assert ws >= 32 * 128 * 2 + 4096 * 4 and L.sfnn_heads_workspace_bytes(ctypes.byref(ok), 8) > ws
    assert L.sfnn_heads_workspace_bytes(ctypes.byref(ok), 0) == 0
    assert L.sfnn_head_qkv(None, fake, 1, fake, fake, None) == 1
    assert L.sfnn_head_qkv(ctypes.byref(ok), fake, 1, None, fake, None) == 1          # no head mask
    for bad in (H(4096, 32, 12, 1, fake, None, fake, None),    # head_dim % 8
                H(4096, 3, 8, 1, fake, None, fake, None),      # n_heads * head_dim % 64
                H(4000, 32, 128, 1, fake, None, fake, None),   # d_model % 128
                H(4096, 1024, 128, 1, fake, None, fake, None)):  # n_heads * head_dim > 65536
        assert L.sfnn_head_qkv(ctypes.byref(bad), fake, 1, fake, fake, None) == 2
        assert L.sfnn_heads_workspace_bytes(ctypes.byref(bad), 1) == 0
    assert L.sfnn_head_qkv(ctypes.byref(H(4096, 32, 128, 2, fake, None, fake, None)), fake, 1, fake, fake,
                           None) == 4                                                 # INT4
    assert L.sfnn_head_qkv(ctypes.byref(ok), fake, 65, fake, fake, None) == 2
    assert L.sfnn_head_qkv(ctypes.byref(ok), fake + 4, 1, fake, fake, None) == 3
    assert L.sfnn_head_out(ctypes.byref(ok), fake, 1, fake, fake, fake, 16, None) == 5


def test_gather_rows_rejects_overlap(L):
    fake = 1 << 20
    perm = 1 << 24
    assert L.sfnn_gather_rows(fake, perm, 64, 256, fake, None) == 2            # in place
    assert L.sfnn_gather_rows(fake, perm, 64, 256, fake + 4096, None) == 2     # dst inside src
    assert L.sfnn_gather_rows(fake + 4096, perm, 64, 256, fake, None) == 2     # src inside dst


def test_layer_noalloc_validation(L):
    """The no-allocation layer call checks its arguments and the scratch limit
    on the host, before any HIP call (so this runs without a GPU)."""
    import activation_sparse_gemv_amd as m
    P, F = m._lib.sfnn_pred, m._lib.sfnn_ffn
    fake = 1 << 20
    assert m.SFNN_NOALLOC_SCRATCH_BYTES == 32 << 20
    hdr = open(os.path.join(ROOT, "include", "sfnn.h")).read()
    assert "#define SFNN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)" in hdr
    # the largest workload (d_model 12288, d_ff 49152, INT4 FFN, fp16 rank-1024
    # predictor): batch 64 needs more than the scratch array holds
    p = P(12288, 49152, 1024, 1, fake, fake, fake)
    f = F(12288, 49152, 2, 0, fake, None, fake, fake, None, fake, None, None, None)
    big = L.sfnn_workspace_bytes(ctypes.byref(p), ctypes.byref(f), 64)
    assert big > m.SFNN_NOALLOC_SCRATCH_BYTES
    assert L.sfnn_layer_noalloc(ctypes.byref(p), ctypes.byref(f), fake, 64, fake, None, None, None, None) == 5
    assert L.sfnn_workspace_bytes(ctypes.byref(p), ctypes.byref(f), 1) <= m.SFNN_NOALLOC_SCRATCH_BYTES
    # the same argument checks as sfnn_layer
    assert L.sfnn_layer_noalloc(None, ctypes.byref(f), fake, 1, fake, None, None, None, None) == 1
    assert L.sfnn_layer_noalloc(ctypes.byref(p), ctypes.byref(f), None, 1, fake, None, None, None, None) == 1
    assert L.sfnn_layer_noalloc(ctypes.byref(p), ctypes.byref(f), fake, 0, fake, None, None, None, None) == 2
    assert L.sfnn_layer_noalloc(ctypes.byref(p), ctypes.byref(f), fake + 4, 1, fake, None, None, None, None) == 3
    q = P(12288, 49152, 1024, 0, fake, fake, fake)     # fp32 predictor with an INT4 (fp16-input) FFN
    assert L.sfnn_layer_noalloc(ctypes.byref(q), ctypes.byref(f), fake, 1, fake, None, None, None, None) == 4


def test_pred_descriptor_layout_matches_header():
    """The ctypes mirror of sfnn_pred ends with hot_prefix and dense_min_batch
    (two int32 after three pointers), as include/sfnn.h declares it."""
    import activation_sparse_gemv_amd as m
    P = m._lib.sfnn_pred
    assert [f[0] for f in P._fields_][-2:] == ["hot_prefix", "dense_min_batch"]
    assert P.dense_min_batch.offset == P.hot_prefix.offset + 4
    assert ctypes.sizeof(P) == 48
    src = open(os.path.join(os.path.dirname(__file__), "..", "include", "sfnn.h")).read()
    body = src[src.index("typedef struct sfnn_pred {"):src.index("} sfnn_pred;")]
    assert body.index("hot_prefix") < body.index("dense_min_batch")


# ---- dense-switch threshold from fire counts (host only) ---------------------

def _enumerated_union_share(p, b):
    """Expected share of neurons touched by b independent tokens, by summing
    over every joint firing outcome (2^(len(p) * b) of them): no closed form."""
    import itertools
    n = len(p)
    total = 0.0
    for bits in itertools.product((0, 1), repeat=n * b):
        prob = 1.0
        for k, on in enumerate(bits):
            pk = p[k % n]
            prob *= pk if on else 1.0 - pk
        touched = sum(1 for i in range(n) if any(bits[t * n + i] for t in range(b)))
        total += prob * touched / n
    return total


def test_dense_min_batch_matches_enumeration(L):
    import activation_sparse_gemv_amd as m
    counts = np.array([2, 1, 3], dtype=np.uint32)   # over 4 tokens: p = 0.5, 0.25, 0.75
    u = [_enumerated_union_share([0.5, 0.25, 0.75], b) for b in (1, 2, 3, 4)]
    assert all(u[k] < u[k + 1] for k in range(3))
    assert abs(u[0] - 0.5) < 1e-12
    for b in range(1, 5):
        lo = u[b - 2] if b > 1 else 0.0
        for c in (lo + 1e-6, (lo + u[b - 1]) / 2, u[b - 1] - 1e-6):
            assert m.sfnn_dense_min_batch(counts, 4, 3, c, 64) == b, (b, c)
    # beyond max_batch: never
    assert m.sfnn_dense_min_batch(counts, 4, 3, (u[2] + u[3]) / 2, 3) == -1


@pytest.mark.parametrize("k,n,c", [(1, 10, 0.45), (1, 20, 0.65), (3, 100, 0.5), (7, 70, 0.9)])
def test_dense_min_batch_uniform_closed_form(L, k, n, c):
    """Every neuron firing with p = k/n: the share after b tokens is
    1 - (1 - p)^b, so the threshold is ceil(log(1 - c) / log(1 - p))."""
    import math
    import activation_sparse_gemv_amd as m
    p = k / n
    want = math.ceil(math.log(1 - c) / math.log(1 - p))
    assert abs(math.log(1 - c) / math.log(1 - p) - round(math.log(1 - c) / math.log(1 - p))) > 1e-6
    counts = np.full(2048, k, dtype=np.uint32)
    assert m.sfnn_dense_min_batch(counts, n, 2048, c, 4096) == want
    assert m.sfnn_dense_min_batch(counts, n, 2048, c, want - 1) == -1


def test_dense_min_batch_special_profiles(L):
    import activation_sparse_gemv_amd as m
    f = 1024
    half = np.zeros(f, dtype=np.uint32)
    half[: f // 2] = 50                      # half always fire, half never: the share is 1/2 at any batch
    assert m.sfnn_dense_min_batch(half, 50, f, 0.5, 1000) == 1
    assert m.sfnn_dense_min_batch(half, 50, f, 0.5001, 1000) == -1
    assert m.sfnn_dense_min_batch(np.zeros(f, dtype=np.uint32), 10, f, 1e-6, 1000) == -1   # nothing fires
    assert m.sfnn_dense_min_batch(np.full(f, 10, dtype=np.uint32), 10, f, 1.0, 1) == 1    # everything fires
    # same mean rate, power law vs uniform: the power law's union grows slower
    rng = np.random.default_rng(5)
    w = 1.0 / np.arange(1, f + 1) ** 0.9
    pz = np.minimum(w * (0.1 * f / w.sum()), 1.0)
    zipf = np.round(pz * 1000).astype(np.uint32)
    uni = np.full(f, int(round(zipf.mean())), dtype=np.uint32)
    rng.shuffle(zipf)
    assert m.sfnn_dense_min_batch(zipf, 1000, f, 0.45, 4096) > m.sfnn_dense_min_batch(uni, 1000, f, 0.45, 4096)


def test_dense_min_batch_rejects_bad_arguments(L):
    c = np.full(64, 3, dtype=np.uint32)
    out = ctypes.c_int32(77)
    cp = c.ctypes.data
    fn = L.sfnn_dense_min_batch
    assert fn(None, 10, 64, ctypes.c_float(0.5), 8, ctypes.byref(out)) == 1
    assert fn(cp, 10, 64, ctypes.c_float(0.5), 8, None) == 1
    for n, f, cr, mb in [(0, 64, 0.5, 8), (10, 0, 0.5, 8), (10, 64, 0.5, 0), (10, 64, 0.0, 8), (10, 64, 1.5, 8),
                         (10, 64, float("nan"), 8), (2, 64, 0.5, 8)]:   # the last: counts 3 > 2 profiled tokens
        assert fn(cp, n, f, ctypes.c_float(cr), mb, ctypes.byref(out)) == 2, (n, f, cr, mb)
    assert out.value == 77
