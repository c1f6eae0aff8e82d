"""GPU parity of the unfused baselines: eager dequantization (bit-exact against
the oracle's dequantized weight rounded once to fp16), the dense fp16 GEMV,
the eager chain end to end, and the separate Tile-COO SpMV."""
import os

import numpy as np
import pytest

import synth
from oracle import reference as ref
from tests.gpu_util import assert_within, dev, host, say, torch

pytestmark = pytest.mark.gpu

q = pytest.importorskip("gemm_unpack_bit_amd")

SHAPES = [(16, 128), (37, 384), (300, 2176), (1000, 640)]


def _uniform_dev(c, bits):
    return q.pack(dev(c["codes"]), bits), dev(c["scales"]), q.pack_zeros(dev(c["zeros"]), bits)


def _bits16(a):
    return np.asarray(a, dtype=np.float16).view(np.uint16)


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("N,K", SHAPES)
def test_dequant_uniform_bit_exact(bits, N, K):
    say("dequant", bits, N, K)
    c = synth.uniform_case(N + K + bits, 1, N, K, bits)
    wq, s, zq = _uniform_dev(c, bits)
    w = host(q.dequant(wq, s, zq, bits, K))
    w_ref = ref.dequant_uniform(c["codes"], c["scales"], c["zeros"]).astype(np.float16)
    assert np.array_equal(_bits16(w), _bits16(w_ref))


@pytest.mark.parametrize("N,K", SHAPES)
def test_dequant_lut4_bit_exact(N, K):
    say("dequant lut4", N, K)
    c = synth.lut4_case(N + 2 * K, 1, N, K)
    w = host(q.dequant_lut4(q.pack(dev(c["codes"]), 4), dev(c["absmax"]), dev(c["lut"]), K))
    w_ref = ref.dequant_lut4(c["codes"], c["absmax"], c["lut"]).astype(np.float16)
    assert np.array_equal(_bits16(w), _bits16(w_ref))


def test_dequant_lut4_signed_zero_table():
    """A table holding +0, -0 and negative levels: the signs of the products
    (including zeros) match the exact product rounded once."""
    N, K = 64, 256
    c = synth.lut4_case(5, 1, N, K)
    lut = c["lut"].copy()
    lut[0], lut[1], lut[7] = 0.0, -0.0, -lut[7]
    w = host(q.dequant_lut4(q.pack(dev(c["codes"]), 4), dev(c["absmax"]), dev(lut), K))
    w_ref = ref.dequant_lut4(c["codes"], c["absmax"], lut).astype(np.float16)
    assert np.array_equal(_bits16(w), _bits16(w_ref))


@pytest.mark.parametrize("N,K", SHAPES + [(2048, 4096)])
@pytest.mark.parametrize("M", [1, 2, 3, 8, 16])
def test_gemv_f16_small_shapes(N, K, M):
    say("gemv_f16", M, N, K)
    c = synth.dense_case(7 * N + K + M, M, N, K)
    y = host(q.gemv_f16(dev(c["x"]), dev(c["w"])))
    y_ref, A = ref.gemv_dense(c["x"], c["w"])
    assert_within(y, y_ref, A, f"gemv_f16 M={M} N={N} K={K}")


@pytest.mark.parametrize("cfg", ["1,8,1", "1,8,3", "1,8,8", "1,4,4", "1,4,8", "2,4,2", "2,4,8", "4,4,5", "4,4,8"])
def test_gemv_f16_every_launch_shape(cfg, monkeypatch):
    """Every accepted (tile rows, chunk, waves) shape on ragged rows and a K
    whose last chunk is partial."""
    for M, N, K in [(5, 300, 2176), (16, 1000, 640), (1, 70, 128)]:
        say("gemv_f16 cfg", cfg, M, N, K)
        c = synth.dense_case(3 * N + K, M, N, K)
        monkeypatch.setenv("QGEMV_DENSE_CFG", cfg)
        y = host(q.gemv_f16(dev(c["x"]), dev(c["w"])))
        monkeypatch.delenv("QGEMV_DENSE_CFG")
        y_ref, A = ref.gemv_dense(c["x"], c["w"])
        assert_within(y, y_ref, A, f"gemv_f16 cfg={cfg} M={M} N={N} K={K}")


def test_gemv_f16_deterministic_and_one_hot():
    """Two calls agree bit for bit; a one-hot x returns the selected weight column."""
    M, N, K = 4, 1000, 4096
    c = synth.dense_case(9, M, N, K)
    x, w = dev(c["x"]), dev(c["w"])
    assert np.array_equal(_bits16(host(q.gemv_f16(x, w))), _bits16(host(q.gemv_f16(x, w))))
    xo = np.zeros((M, K), np.float16)
    for m, k in enumerate([0, 127, 2048, 4095]):
        xo[m, k] = 1.0
    y = host(q.gemv_f16(dev(xo), w))
    expect = c["w"][:, [0, 127, 2048, 4095]].T
    assert np.array_equal(_bits16(y), _bits16(expect))


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("M", [1, 4])
def test_eager_chain_matches_uniform_oracle(bits, M):
    N, K = 300, 2176
    say("eager chain", bits, M)
    c = synth.uniform_case(31 + bits + M, M, N, K, bits)
    wq, s, zq = _uniform_dev(c, bits)
    y = host(q.gemv_f16(dev(c["x"]), q.dequant(wq, s, zq, bits, K)))
    y_ref, A = ref.gemv_uniform(c["x"], c["codes"], c["scales"], c["zeros"])
    assert_within(y, y_ref, A, f"eager W{bits} M={M}")


def test_eager_lut4_chain_matches_oracle():
    N, K, M = 300, 2176, 2
    say("eager lut4 chain")
    c = synth.lut4_case(33, M, N, K)
    w = q.dequant_lut4(q.pack(dev(c["codes"]), 4), dev(c["absmax"]), dev(c["lut"]), K)
    y = host(q.gemv_f16(dev(c["x"]), w))
    y_ref, A = ref.gemv_lut4(c["x"], c["codes"], c["absmax"], c["lut"])
    assert_within(y, y_ref, A, "eager lut4")


def _tilecoo_dev(c, N, K):
    ptr, rec = q.tilecoo_encode(N, K, c["o_rows"], c["o_cols"], c["o_vals"])
    return dev(ptr.view(np.int32)), dev(rec.view(np.int32))


@pytest.mark.parametrize("N,K,frac", [(16, 128, 0.05), (100, 384, 0.02), (300, 2176, 0.005), (1000, 640, 0.01),
                                      (48, 1024, 0.3)])
@pytest.mark.parametrize("M", [1, 3, 16])
def test_spmv_adds_outliers(N, K, frac, M):
    say("spmv", M, N, K, frac)
    c = synth.outlier_case(N * 5 + K + M, M, N, K, frac=frac)
    yp = synth.output_prior(N + M, M, N)
    tp, tr = _tilecoo_dev(c, N, K)
    y = host(q.spmv_tilecoo(dev(c["x"]), tp, tr, dev(yp)))
    y_ref, A = ref.add_sparse(yp, c["x"], c["o_rows"], c["o_cols"], c["o_vals"])
    assert_within(y, y_ref, A, f"spmv M={M} N={N} K={K} frac={frac}")
    untouched = np.setdiff1d(np.arange(N), c["o_rows"])
    assert np.array_equal(_bits16(y[:, untouched]), _bits16(yp[:, untouched]))


def test_spmv_without_outliers_leaves_y():
    N, K = 200, 512
    say("spmv nnz=0")
    c = synth.dense_case(3, 2, N, K)
    yp = synth.output_prior(4, 2, N)
    ptr, _ = q.tilecoo_encode(N, K, [], [], [])
    y = host(q.spmv_tilecoo(dev(c["x"]), dev(ptr.view(np.int32)), None, dev(yp)))
    assert np.array_equal(_bits16(y), _bits16(yp))


@pytest.mark.parametrize("M", [1, 4])
def test_unfused_outlier_chain_matches_oracle(M):
    """The dense W4 kernel, then the separate SpMV on its output."""
    N, K = 1000, 2176
    say("unfused outlier chain", M)
    c = synth.outlier_case(41 + M, M, N, K)
    wq, s, zq = _uniform_dev(c, 4)
    tp, tr = _tilecoo_dev(c, N, K)
    x = dev(c["x"])
    y = host(q.spmv_tilecoo(x, tp, tr, q.w4a16(x, wq, s, zq)))
    y_ref, A = ref.gemv_outlier(c["x"], c["codes"], c["scales"], c["zeros"], c["o_rows"], c["o_cols"], c["o_vals"])
    assert_within(y, y_ref, A, f"unfused outlier M={M}")


# -- full sizes, in the launch configurations the benchmark times, on sampled rows

def _sample(N):
    rng = np.random.default_rng(N)
    return np.unique(np.concatenate([[0, 1, 15, 16, N // 2, N - 16, N - 1], rng.integers(0, N, 25)]))


def test_full_size_eager_w4_gate_up():
    N, K, M = 28672, 4096, 1
    say("full eager w4", N, K)
    c = synth.uniform_case(51, M, N, K, 4)
    wq, s, zq = _uniform_dev(c, 4)
    w = q.dequant(wq, s, zq, 4, K)
    y = host(q.gemv_f16(dev(c["x"]), w))
    rows = _sample(N)
    w_rows = host(w[torch().from_numpy(rows).cuda()])
    w_ref = ref.dequant_uniform(c["codes"][rows], c["scales"][rows], c["zeros"][rows]).astype(np.float16)
    assert np.array_equal(_bits16(w_rows), _bits16(w_ref))
    y_ref, A = ref.gemv_uniform(c["x"], c["codes"], c["scales"], c["zeros"], rows=rows)
    assert_within(y[:, rows], y_ref, A, "full eager w4 gate_up")


def test_full_size_eager_lut4_down():
    N, K, M = 4096, 14336, 1
    say("full eager lut4", N, K)
    c = synth.lut4_case(52, M, N, K)
    w = q.dequant_lut4(q.pack(dev(c["codes"]), 4), dev(c["absmax"]), dev(c["lut"]), K)
    y = host(q.gemv_f16(dev(c["x"]), w))
    rows = _sample(N)
    y_ref, A = ref.gemv_lut4(c["x"], c["codes"], c["absmax"], c["lut"], rows=rows)
    assert_within(y[:, rows], y_ref, A, "full eager lut4 down")


def test_full_size_unfused_outlier_gate_up():
    N, K, M = 28672, 4096, 1
    say("full unfused outlier", N, K)
    c = synth.outlier_case(53, M, N, K)
    wq, s, zq = _uniform_dev(c, 4)
    tp, tr = _tilecoo_dev(c, N, K)
    x = dev(c["x"])
    y = host(q.spmv_tilecoo(x, tp, tr, q.w4a16(x, wq, s, zq)))
    rows = _sample(N)
    y_ref, A = ref.gemv_outlier(c["x"], c["codes"], c["scales"], c["zeros"], c["o_rows"], c["o_cols"],
                                c["o_vals"], rows=rows)
    assert_within(y[:, rows], y_ref, A, "full unfused outlier gate_up")
