"""Pins of the plain C oracle (oracle/cref.c) against the float64 numpy
oracle, exact rational brute force and closed forms (CPU only)."""
import numpy as np
import pytest

import synth
from oracle import cref, exact, reference as ref


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("M,N,K", [(1, 5, 128), (3, 17, 384), (2, 64, 1024)])
def test_matches_numpy_oracle(bits, M, N, K):
    c = synth.uniform_case(900 + N + bits, M, N, K, bits)
    y, A = cref.gemv_uniform(c["x"], c["codes"], c["scales"], c["zeros"], bits)
    y0, A0 = ref.gemv_uniform(c["x"], c["codes"], c["scales"], c["zeros"])
    assert np.allclose(y, y0, rtol=0, atol=1e-12 * max(1.0, float(A0.max())))
    assert np.allclose(A, A0, rtol=1e-14, atol=0)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_matches_exact_brute_force(bits):
    c = synth.uniform_case(910 + bits, 2, 4, 256, bits)
    y, _ = cref.gemv_uniform(c["x"], c["codes"], c["scales"], c["zeros"], bits)
    ye = exact.to_f64(exact.gemv_uniform_exact(c["x"], c["codes"], c["scales"], c["zeros"]))
    assert np.allclose(y, ye, rtol=1e-15, atol=1e-300)


def test_row_range_threads_and_special_cases():
    bits, M, N, K = 4, 2, 40, 512
    c = synth.uniform_case(920, M, N, K, bits)
    full, _ = cref.gemv_uniform(c["x"], c["codes"], c["scales"], c["zeros"], bits, threads=3)
    part, _ = cref.gemv_uniform(c["x"], c["codes"], c["scales"], c["zeros"], bits, rows=(7, 23), threads=1)
    assert np.array_equal(part, full[:, 7:23])
    # q == z gives exactly 0; one-hot x gives one dequantized weight exactly
    zc = synth.degenerate_codes(920, c["zeros"], bits)
    y0, A0 = cref.gemv_uniform(c["x"], zc, c["scales"], c["zeros"], bits)
    assert np.all(y0 == 0.0) and np.all(A0 == 0.0)
    x = np.zeros((1, K), dtype=np.float16)
    x[0, 300] = 1.0
    y1, _ = cref.gemv_uniform(x, c["codes"], c["scales"], c["zeros"], bits)
    w = c["scales"][:, 2].astype(np.float64) * (c["codes"][:, 300].astype(np.float64) - c["zeros"][:, 2])
    assert np.array_equal(y1[0], w)


def test_fp16_decoding_specials():
    """Subnormal, largest normal, infinities and NaN activations decode exactly."""
    bits, N, K = 8, 3, 128
    codes = np.full((N, K), 1, dtype=np.uint8)
    zeros = np.zeros((N, 1), dtype=np.uint8)
    scales = np.ones((N, 1), dtype=np.float16)
    for v in (2.0 ** -24, 6.097555160522461e-05, 65504.0, -65504.0):
        x = np.zeros((1, K), dtype=np.float16)
        x[0, 5] = v
        y, _ = cref.gemv_uniform(x, codes, scales, zeros, bits)
        assert np.all(y == float(np.float16(v)))
    x = np.zeros((1, K), dtype=np.float16)
    x[0, 0] = np.inf
    assert np.all(np.isinf(cref.gemv_uniform(x, codes, scales, zeros, bits)[0]))
    x[0, 0] = np.nan
    assert np.all(np.isnan(cref.gemv_uniform(x, codes, scales, zeros, bits)[0]))


def test_rejects_bad_arguments():
    c = synth.uniform_case(930, 1, 4, 128, 4)
    with pytest.raises(ValueError):
        cref.gemv_uniform(c["x"], c["codes"], c["scales"], c["zeros"], 3)
    with pytest.raises(ValueError):
        cref.gemv_uniform(c["x"], c["codes"], c["scales"], c["zeros"], 4, rows=(2, 9))
