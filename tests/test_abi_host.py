"""Host-side checks of the C-ABI library (no GPU needed): it loads, exports
every symbol the header declares, validates arguments before launching, and
the host-only hot-first ordering matches the oracle's."""
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
    assert m.sfnn_version() >= 340  # 340: sfnn_pred.dense_min_batch
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
