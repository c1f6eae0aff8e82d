"""GPU parity of the fused outlier-aware W4A16 variant (dense uniform W4 +
fp16 Tile-COO outliers in one kernel) against the float64 oracle."""
import numpy as np
import pytest

import synth
from oracle import reference as ref
from tests.gpu_util import assert_within, dev, host, sample_rows, say, torch

pytestmark = pytest.mark.gpu

q = pytest.importorskip("gemm_unpack_bit_amd")
PATHS = [q.PATH_AUTO, q.PATH_VALU, q.PATH_MFMA]


def _upload(c, N, K):
    wq = q.pack(dev(c["codes"]), 4)
    zq = q.pack_zeros(dev(c["zeros"]), 4)
    ptr, rec = q.tilecoo_encode(N, K, c["o_rows"], c["o_cols"], c["o_vals"])
    return wq, dev(c["scales"]), zq, dev(ptr.view(np.int32)), dev(rec.view(np.int32))


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("N,K,frac", [(16, 128, 0.05), (100, 384, 0.02), (256, 1024, 0.01), (300, 2176, 0.005),
                                      (1000, 640, 0.01)])
@pytest.mark.parametrize("M", [1, 2, 5, 16])
def test_outlier_small_shapes(path, N, K, frac, M):
    say("outlier", path, N, K, frac, M)
    c = synth.outlier_case(N * 3 + K, M, N, K, frac=frac)
    wq, s, zq, tp, tr = _upload(c, N, K)
    y = host(q.outlier(dev(c["x"]), wq, s, zq, tp, tr, path))
    y_ref, A = ref.gemv_outlier(c["x"], c["codes"], c["scales"], c["zeros"], c["o_rows"], c["o_cols"], c["o_vals"])
    assert_within(y, y_ref, A, f"outlier M={M} N={N} K={K} path={path}")


@pytest.mark.parametrize("path", [q.PATH_VALU, q.PATH_MFMA])
def test_no_outliers_equals_dense_bitwise(path):
    """nnz = 0: the same dense kernel path, so y equals qgemv_uniform bit for bit."""
    say("outlier nnz=0", path)
    N, K, M = 4096, 4096, 1 if path == q.PATH_VALU else 4
    c = synth.uniform_case(3, M, N, K, 4)
    wq = q.pack(dev(c["codes"]), 4)
    zq = q.pack_zeros(dev(c["zeros"]), 4)
    s, x = dev(c["scales"]), dev(c["x"])
    ptr, rec = q.tilecoo_encode(N, K, [], [], [])
    t = torch()
    y = host(q.outlier(x, wq, s, zq, dev(ptr.view(np.int32)), t.zeros(0, dtype=t.int32, device="cuda"), path))
    yd = host(q.uniform(x, wq, s, zq, 4, path))
    assert np.array_equal(y.view(np.uint16), yd.view(np.uint16))


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("N,K", [(256, 1024), (4096, 4096), (28672, 4096)])
def test_degenerate_dense_part(path, N, K):
    """Dense codes equal to their zero points (the dense part is exactly 0):
    with no outliers y = 0 exactly; with outliers y = the sparse product
    alone, within the bound of that product's A.  Every engine, M = 1, 2, 4."""
    c = synth.outlier_case(31 + N, 4, N, K)
    codes = synth.degenerate_codes(32, c["zeros"], 4)
    wq, zq, s = q.pack(dev(codes), 4), q.pack_zeros(dev(c["zeros"]), 4), dev(c["scales"])
    ptr0, _ = q.tilecoo_encode(N, K, [], [], [])
    ptr, rec = q.tilecoo_encode(N, K, c["o_rows"], c["o_cols"], c["o_vals"])
    t = torch()
    empty = t.zeros(0, dtype=t.int32, device="cuda")
    ys, As = ref.gemv_outlier(c["x"], codes, c["scales"], c["zeros"], c["o_rows"], c["o_cols"], c["o_vals"])
    for M in (1, 2, 4):
        say("outlier q==z", path, N, K, M)
        x = dev(c["x"][:M])
        y0 = host(q.outlier(x, wq, s, zq, dev(ptr0.view(np.int32)), empty, path))
        assert np.all(y0.astype(np.float64) == 0.0), f"q==z, no outliers, M={M} path={path}"
        y = host(q.outlier(x, wq, s, zq, dev(ptr.view(np.int32)), dev(rec.view(np.int32)), path))
        assert_within(y, ys[:M], As[:M], f"q==z plus outliers M={M} N={N} K={K} path={path}")


def test_zero_scales_give_pure_sparse_product():
    """s = 0: the dense part vanishes and y = S x exactly up to fp32 summation."""
    say("outlier spmv")
    N, K = 384, 1024
    c = synth.outlier_case(11, 2, N, K, frac=0.02)
    c["scales"][:] = 0
    wq, s, zq, tp, tr = _upload(c, N, K)
    y = host(q.outlier(dev(c["x"]), wq, s, zq, tp, tr))
    ys, As = ref.sparse_part(c["x"], N, c["o_rows"], c["o_cols"], c["o_vals"])
    assert_within(y, ys, As, "outlier pure sparse")


def test_single_outlier_one_hot_exact():
    """One outlier at (r, k) and x = e_k: y[r] = fp16(s (q - z) + v) exactly here
    (both terms are exact in fp32 and their sum is exact for these values)."""
    say("outlier one-hot")
    N, K = 256, 512
    c = synth.uniform_case(5, 1, N, K, 4)
    r, k = 37, 300
    c["o_rows"], c["o_cols"] = np.array([r]), np.array([k])
    c["o_vals"] = np.array([0.5], dtype=np.float16)
    c["scales"][:] = np.float16(0.015625)
    wq, s, zq, tp, tr = _upload(c, N, K)
    x = np.zeros((1, K), dtype=np.float16)
    x[0, k] = 2.0
    y = host(q.outlier(dev(x), wq, s, zq, tp, tr))
    y_ref, _ = ref.gemv_outlier(x, c["codes"], c["scales"], c["zeros"], c["o_rows"], c["o_cols"], c["o_vals"])
    assert np.array_equal(y.view(np.uint16), synth.f16(y_ref).view(np.uint16))


def test_outlier_deterministic():
    say("outlier determinism")
    N, K = 4096, 4096
    c = synth.outlier_case(21, 1, N, K)
    wq, s, zq, tp, tr = _upload(c, N, K)
    x = dev(c["x"])
    y1 = host(q.outlier(x, wq, s, zq, tp, tr))
    y2 = host(q.outlier(x, wq, s, zq, tp, tr))
    assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))


@pytest.mark.parametrize("M", [1, 4, 16])
def test_outlier_4096_config(M):
    """The 4096 x 4096 workload: 0.5% unique outliers ~ N(0, 0.2), every row checked."""
    say("outlier 4096", M)
    N = K = 4096
    c = synth.outlier_case(synth.seed_for(4, 0), M, N, K)
    wq, s, zq, tp, tr = _upload(c, N, K)
    y = host(q.outlier(dev(c["x"]), wq, s, zq, tp, tr))
    y_ref, A = ref.gemv_outlier(c["x"], c["codes"], c["scales"], c["zeros"], c["o_rows"], c["o_cols"], c["o_vals"])
    assert_within(y, y_ref, A, f"outlier 4096 M={M}")


def test_outlier_dense_tiles():
    """Many outliers in one tile (a tile run longer than a staged chunk)."""
    say("outlier dense tile")
    N, K = 128, 256
    c = synth.uniform_case(8, 1, N, K, 4)
    rr, cc = np.meshgrid(np.arange(128), np.arange(128), indexing="ij")
    c["o_rows"], c["o_cols"] = rr.ravel(), cc.ravel() + 128
    c["o_vals"] = synth.f16(synth.normal(8, synth.S_OVAL, 128 * 128, 0.2))
    wq, s, zq, tp, tr = _upload(c, N, K)
    y = host(q.outlier(dev(c["x"]), wq, s, zq, tp, tr))
    y_ref, A = ref.gemv_outlier(c["x"], c["codes"], c["scales"], c["zeros"], c["o_rows"], c["o_cols"], c["o_vals"])
    assert_within(y, y_ref, A, "outlier dense tile")


@pytest.mark.parametrize("path,M", [(q.PATH_VALU, 1), (q.PATH_VALU, 2), (q.PATH_MFMA, 5)])
@pytest.mark.parametrize("N,K", [(300, 2176), (64, 4096)])
def test_outlier_every_launch_shape(monkeypatch, path, M, N, K):
    """Every launch shape the outlier kernel takes, forced through
    QGEMV_OUTLIER_CFG: few waves give a wave more tiles than it prefetches
    records for; ragged N puts outliers in a partial tile-row."""
    say("outlier launch shapes", path, M, N, K)
    c = synth.outlier_case(N + K + M, M, N, K, frac=0.01)
    extra = [(N - 1, 5), (N - 1, K - 1), (0, K - 1)]  # last row and last column
    have = set(zip(c["o_rows"].tolist(), c["o_cols"].tolist()))
    add = [rc for rc in extra if rc not in have]
    if add:
        c["o_rows"] = np.concatenate([c["o_rows"], np.array([r for r, _ in add], dtype=np.int32)])
        c["o_cols"] = np.concatenate([c["o_cols"], np.array([k for _, k in add], dtype=np.int32)])
        c["o_vals"] = np.concatenate([c["o_vals"], np.full(len(add), 0.75, dtype=np.float16)])
    wq, s, zq, tp, tr = _upload(c, N, K)
    x = dev(c["x"])
    y_ref, A = ref.gemv_outlier(c["x"], c["codes"], c["scales"], c["zeros"], c["o_rows"], c["o_cols"], c["o_vals"])
    ran = []
    for tpw, v in ((1, 3), (1, 4), (2, 0)):
        for wk in (1, 2, 4, 8, 16):
            for mt in ((1, 2) if path == q.PATH_VALU else (1,)):
                cfg = f"{tpw},{wk},{mt},{v}"
                monkeypatch.setenv("QGEMV_OUTLIER_CFG", cfg)
                try:
                    y = host(q.outlier(x, wq, s, zq, tp, tr, path))
                except q.QgemvError:
                    continue
                assert_within(y, y_ref, A, f"outlier M={M} N={N} K={K} path={path} cfg={cfg}")
                ran.append(cfg)
    assert len(ran) >= 8, ran


@pytest.mark.parametrize("xlds,plds", [("", "1"), ("0", "1"), ("", "0"), ("0", "0")])
@pytest.mark.parametrize("N,K", [(300, 2176), (64, 4096), (272, 33024)])
def test_outlier_early_batch_every_staging(monkeypatch, xlds, plds, N, K):
    """The VALU engine at one batch row runs a wave's first record batch
    inside the dense loop, behind a wait whose count depends on the loads a
    stage issues: activations staged in LDS or loaded per chunk, quant params
    staged or loaded per lane.  Every combination, every launch shape, with
    enough records per tile-row that waves hold several batches (K = 33024:
    activations too long to stage)."""
    say("outlier early batch", xlds, plds, N, K)
    c = synth.outlier_case(N + K + 7, 1, N, K, frac=0.02)
    wq, s, zq, tp, tr = _upload(c, N, K)
    x = dev(c["x"])
    y_ref, A = ref.gemv_outlier(c["x"], c["codes"], c["scales"], c["zeros"], c["o_rows"], c["o_cols"], c["o_vals"])
    if xlds:
        monkeypatch.setenv("QGEMV_XLDS_MAX", xlds)
    monkeypatch.setenv("QGEMV_PLDS", plds)
    ran = []
    for tpw, v in ((1, 3), (2, 0)):
        for wk in (1, 4, 16):
            cfg = f"{tpw},{wk},1,{v}"
            monkeypatch.setenv("QGEMV_OUTLIER_CFG", cfg)
            try:
                y = host(q.outlier(x, wq, s, zq, tp, tr, q.PATH_VALU))
            except q.QgemvError:
                continue
            assert_within(y, y_ref, A, f"outlier early batch N={N} K={K} cfg={cfg} xlds={xlds} plds={plds}")
            ran.append(cfg)
    assert len(ran) >= 4, ran


@pytest.mark.parametrize("form", ["fused", "split"])
@pytest.mark.parametrize("path", [q.PATH_VALU, q.PATH_MFMA])
@pytest.mark.parametrize("M", [1, 5, 16])
def test_outlier_both_forms(monkeypatch, form, path, M):
    """The fused kernel and the dense-then-sparse sequence the call takes on
    wide layers, each forced through QGEMV_OUTLIER_FORM, on a ragged shape."""
    N, K = 1000, 2176
    say("outlier form", form, path, M)
    c = synth.outlier_case(71 + M, M, N, K, frac=0.01)
    wq, s, zq, tp, tr = _upload(c, N, K)
    monkeypatch.setenv("QGEMV_OUTLIER_FORM", form)
    y = host(q.outlier(dev(c["x"]), wq, s, zq, tp, tr, path))
    y_ref, A = ref.gemv_outlier(c["x"], c["codes"], c["scales"], c["zeros"], c["o_rows"], c["o_cols"], c["o_vals"])
    assert_within(y, y_ref, A, f"outlier form={form} M={M} path={path}")


# -- the decoder-layer shapes at every batch size (sampled rows): long K with
# staged batch rows must still fit the launch's LDS
@pytest.mark.parametrize("N,K,M", [(4096, 14336, 2), (4096, 14336, 4), (4096, 14336, 16), (6144, 4096, 2),
                                   (28672, 4096, 4), (28672, 4096, 16), (8192, 28672, 2)])
def test_outlier_layer_shapes_batched(N, K, M):
    say("outlier layer", N, K, M)
    c = synth.outlier_case(61 + M, M, N, K)
    wq, s, zq, tp, tr = _upload(c, N, K)
    y = host(q.outlier(dev(c["x"]), wq, s, zq, tp, tr))
    rows = sample_rows(N)
    y_ref, A = ref.gemv_outlier(c["x"], c["codes"], c["scales"], c["zeros"], c["o_rows"], c["o_cols"], c["o_vals"],
                                rows=rows)
    assert_within(y[:, rows], y_ref, A, f"outlier M={M} N={N} K={K}")


@pytest.mark.parametrize("path", [q.PATH_VALU, q.PATH_MFMA])
@pytest.mark.parametrize("N,K,M", [(4096, 4096, 1), (28672, 4096, 1), (10240, 8192, 1), (4096, 4096, 2)])
def test_whole_ring_rounds_kernel_equals_general(monkeypatch, path, N, K, M):
    """The fused outlier kernel where K/128 fills whole rounds of its chunk
    ring (QGEMV_FULL_ROUNDS=1, the default) against the general kernel:
    the same y bit for bit."""
    c = synth.outlier_case(800 + N + M, M, N, K)
    wq, s, zq, tp, tr = _upload(c, N, K)
    x = dev(c["x"])
    ys = {}
    for full in ("0", "1"):
        say("outlier full rounds", full, path, N, K, M)
        monkeypatch.setenv("QGEMV_FULL_ROUNDS", full)
        ys[full] = host(q.outlier(x, wq, s, zq, tp, tr, path))
    assert np.array_equal(ys["0"].view(np.uint16), ys["1"].view(np.uint16))
