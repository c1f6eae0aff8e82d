"""GPU parity of the prefill-size GEMM (any M, matrix cores) against the
float64 oracle of the uniform format."""
import numpy as np
import pytest

import synth
from oracle import reference as ref
from tests.gpu_util import assert_within, dev, host, sample_rows, say

pytestmark = pytest.mark.gpu

q = pytest.importorskip("gemm_unpack_bit_amd")


def _case(seed, M, N, K, bits):
    c = synth.uniform_case(seed, M, N, K, bits)
    return c, q.pack(dev(c["codes"]), bits), dev(c["scales"]), q.pack_zeros(dev(c["zeros"]), bits)


# block shapes: (activation tiles, tile-rows per wave, K halves per
# workgroup) = 32 or 64 activation rows x 256 or 128 weight rows, all of K or
# two interleaved halves of it (128-column blocks and K/128 even only: the
# other shapes run one half)
@pytest.mark.parametrize("mi,nt,kh", [("2", "4", "1"), ("4", "4", "1"), ("2", "2", "1"), ("4", "2", "1"),
                                      ("2", "2", "2"), ("4", "2", "2")])
@pytest.mark.parametrize("force", ["0", "1"])  # "1": the GEMM kernel also for M <= 64
@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("M,N,K", [(1, 16, 128), (17, 70, 384), (64, 300, 2048), (100, 1000, 640), (300, 48, 128),
                                   (130, 257, 1152), (96, 200, 1024), (40, 130, 256)])
def test_gemm_small_shapes(bits, M, N, K, force, mi, nt, kh, monkeypatch):
    say("gemm", bits, M, N, K, force, mi, nt, kh)
    monkeypatch.setenv("QGEMV_GEMM_KERNEL", force)
    monkeypatch.setenv("QGEMV_GEMM_MI", mi)
    monkeypatch.setenv("QGEMV_GEMM_NT", nt)
    monkeypatch.setenv("QGEMV_GEMM_KH", kh)
    c, wq, s, zq = _case(M * 7 + N + K + bits, M, N, K, bits)
    y = host(q.gemm_uniform(dev(c["x"]), wq, s, zq, bits))
    y_ref, A = ref.gemv_uniform(c["x"], c["codes"], c["scales"], c["zeros"])
    assert_within(y, y_ref, A, f"gemm W{bits} M={M} N={N} K={K}")


def test_gemm_agrees_with_gemv_and_is_deterministic():
    M, N, K = 16, 1000, 4096
    say("gemm vs gemv")
    c, wq, s, zq = _case(5, M, N, K, 4)
    x = dev(c["x"])
    y1 = host(q.gemm_uniform(x, wq, s, zq, 4))
    y2 = host(q.gemm_uniform(x, wq, s, zq, 4))
    assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))
    yv = host(q.uniform(x, wq, s, zq, 4))
    y_ref, A = ref.gemv_uniform(c["x"], c["codes"], c["scales"], c["zeros"])
    assert_within(y1, y_ref, A, "gemm")
    assert_within(yv, y_ref, A, "gemv")


@pytest.mark.parametrize("kh", ["1", "2"])
@pytest.mark.parametrize("M,N,K", [(512, 4096, 4096), (200, 4096, 14336), (512, 4096, 14336)])
def test_gemm_full_size_sampled(M, N, K, kh, monkeypatch):
    say("gemm full", M, N, K, kh)
    monkeypatch.setenv("QGEMV_GEMM_KH", kh)
    c, wq, s, zq = _case(6 + M, M, N, K, 4)
    y = host(q.gemm_uniform(dev(c["x"]), wq, s, zq, 4))
    rows = sample_rows(N)
    y_ref, A = ref.gemv_uniform(c["x"], c["codes"], c["scales"], c["zeros"], rows=rows)
    assert_within(y[:, rows], y_ref, A, f"gemm full M={M} N={N} K={K}")
