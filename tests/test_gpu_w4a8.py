"""GPU parity of the W4A8 GEMV (int8 activations with one symmetric scale per
row, 4-bit weights padded to int8, int8 matrix cores) against the oracle."""
import numpy as np
import pytest

import synth
from oracle import reference as ref
from tests.gpu_util import assert_within, dev, host, sample_rows, say, torch

pytestmark = pytest.mark.gpu

q = pytest.importorskip("gemm_unpack_bit_amd")


def _run(x, c, wk=None, monkeypatch=None):
    t = torch()
    M, K = x.shape
    ws = t.zeros(q.w4a8_workspace_bytes(M, K), dtype=t.uint8, device="cuda")
    if wk is not None:
        monkeypatch.setenv("QGEMV_W4A8_WK", str(wk))
    y = host(q.w4a8(dev(x), q.pack(dev(c["codes"]), 4), dev(c["scales"]), q.pack_zeros(dev(c["zeros"]), 4), ws))
    w = host(ws)
    xq = w[:M * K].view(np.int8).reshape(M, K)
    off = (M * K + 15) // 16 * 16
    sx = w[off:off + 4 * M].view(np.float32)
    return y, xq, sx


# the quantization takes 2048 k per workgroup: K = 32768 is 16 whole parts, 33024 ends in a short one
@pytest.mark.parametrize("M,N,K", [(1, 16, 128), (3, 70, 384), (16, 300, 2048), (5, 1000, 640), (2, 48, 14336),
                                   (1, 24, 32768), (3, 40, 33024)])
def test_w4a8_matches_oracle_and_quantizes_exactly(M, N, K):
    say("w4a8", M, N, K)
    c = synth.uniform_case(N + K + M, M, N, K, 4)
    x = c["x"].copy()
    if M >= 3:
        x[1] = 0                                    # a zero row
        x[2, :4] = [np.float16(-65504.0), 1.0, 0.5, 0.25]  # an extreme row
    y, xq, sx = _run(x, c)
    q_ref, s_ref = ref.quantize_activations_int8(x)
    assert np.array_equal(xq, q_ref) and np.array_equal(sx.view(np.uint32), s_ref.view(np.uint32))
    y_ref, A = ref.gemv_w4a8(x, c["codes"], c["scales"], c["zeros"])
    assert_within(y, y_ref, A, f"w4a8 M={M} N={N} K={K}")


def test_w4a8_ties_round_to_even():
    """x / s landing on k + 0.5 rounds to the even integer (max |x| = 2)."""
    M, N, K = 1, 64, 128
    c = synth.uniform_case(3, M, N, K, 4)
    x = np.zeros((M, K), np.float16)
    x[0, :4] = [2.0, 1.0, -1.0, np.float16(3.0 / 127.0)]  # 127, 63.5 -> 64, -63.5 -> -64, 1.5 -> 2
    y, xq, sx = _run(x, c)
    q_ref, _ = ref.quantize_activations_int8(x)
    assert np.array_equal(xq, q_ref)
    assert xq[0, :3].tolist() == [127, 64, -64]


@pytest.mark.parametrize("wk", [1, 3, 8, 16])
@pytest.mark.parametrize("M", [1, 4])
def test_w4a8_every_wave_count(wk, M, monkeypatch):
    """Every wave count, including runs past the group count and idle waves."""
    N, K = 200, 2048
    say("w4a8 wk", wk, M)
    c = synth.uniform_case(7 + wk + M, M, N, K, 4)
    y, xq, _ = _run(c["x"], c, wk, monkeypatch)
    assert np.array_equal(xq, ref.quantize_activations_int8(c["x"])[0])
    y_ref, A = ref.gemv_w4a8(c["x"], c["codes"], c["scales"], c["zeros"])
    assert_within(y, y_ref, A, f"w4a8 wk={wk} M={M}")


# the launch configurations the benchmark times (M = 16 on gate+up and qkv: two tile-rows per workgroup)
@pytest.mark.parametrize("M,N,K", [(1, 28672, 4096), (1, 4096, 14336), (4, 4096, 14336), (16, 28672, 4096),
                                   (16, 6144, 4096), (16, 4096, 14336)])
def test_w4a8_full_size_sampled(M, N, K):
    say("w4a8 full", M, N, K)
    c = synth.uniform_case(8 + M, M, N, K, 4)
    y, _, _ = _run(c["x"], c)
    rows = sample_rows(N)
    y_ref, A = ref.gemv_w4a8(c["x"], c["codes"], c["scales"], c["zeros"], rows=rows)
    assert_within(y[:, rows], y_ref, A, f"w4a8 full M={M} N={N} K={K}")


def test_w4a8_deterministic():
    M, N, K = 8, 1000, 4096
    c = synth.uniform_case(9, M, N, K, 4)
    y1, _, _ = _run(c["x"], c)
    y2, _, _ = _run(c["x"], c)
    assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))


@pytest.mark.parametrize("tr", [1, 2])
@pytest.mark.parametrize("M,N,K", [(1, 1000, 640), (16, 300, 2048), (6, 8200, 1024), (16, 8208, 384)])
def test_w4a8_tile_rows_per_workgroup(tr, M, N, K, monkeypatch):
    """One or two tile-rows per workgroup (two share each activation load),
    forced through QGEMV_W4A8_TR, on odd tile-row counts and ragged rows."""
    say("w4a8 tr", tr, M, N, K)
    monkeypatch.setenv("QGEMV_W4A8_TR", str(tr))
    c = synth.uniform_case(11 * tr + M + N, M, N, K, 4)
    y, xq, _ = _run(c["x"], c)
    assert np.array_equal(xq, ref.quantize_activations_int8(c["x"])[0])
    y_ref, A = ref.gemv_w4a8(c["x"], c["codes"], c["scales"], c["zeros"])
    assert_within(y, y_ref, A, f"w4a8 tr={tr} M={M} N={N} K={K}")
