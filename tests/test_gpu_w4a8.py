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


# ----------------------------------------------------------------------------
# the split strategy (two 4-bit activation slices on the fp8 matrix cores) and
# asymmetric activations (zero points on both operands, expansion)
# ----------------------------------------------------------------------------
def _e4m3(v):
    """OCP fp8 e4m3 byte of a small integer (|v| <= 128), written from the
    format's definition (bias 7, 3 mantissa bits); None if v needs more than
    4 significant bits."""
    v = int(v)
    if v == 0:
        return 0
    s = 0x80 if v < 0 else 0
    a = abs(v)
    e = a.bit_length() - 1
    m = (a << 3 >> e) & 7
    if (8 + m) << e >> 3 != a:
        return None
    return s | ((e + 7) << 3) | m


# indexed by v + 128; 0xFF (a NaN pattern no slice can produce) where v is not exact
_E4M3 = np.array([0xFF if _e4m3(v) is None else _e4m3(v) for v in range(-128, 128)], dtype=np.uint8)


def _packed(c):
    return q.pack(dev(c["codes"]), 4), dev(c["scales"]), q.pack_zeros(dev(c["zeros"]), 4)


SPLIT_SHAPES = [(1, 16, 128), (3, 70, 384), (16, 300, 2048), (5, 1000, 640), (2, 48, 14336), (3, 40, 33024),
                (1, 28672, 4096), (16, 4096, 14336), (16, 6144, 4096)]


@pytest.mark.parametrize("M,N,K", SPLIT_SHAPES)
def test_w4a8_split_equals_padding_bitwise(M, N, K):
    """The split strategy reconstructs the same exact integer group sums as
    padding, so y is the same bits; its slices are the exact decomposition
    of the padding strategy's x_q, as fp8 e4m3."""
    say("w4a8 split", M, N, K)
    t = torch()
    c = synth.uniform_case(N + K + 2 * M, M, N, K, 4)
    x = c["x"].copy()
    if M >= 3:
        x[1] = 0
        x[2, :4] = [np.float16(-65504.0), 1.0, 0.5, 0.25]
    xd, (wq, s, zq) = dev(x), _packed(c)
    ws = t.zeros(q.w4a8_split_workspace_bytes(M, K), dtype=t.uint8, device="cuda")
    y = host(q.w4a8_split(xd, wq, s, zq, ws))
    wsp = t.zeros(q.w4a8_workspace_bytes(M, K), dtype=t.uint8, device="cuda")
    yp = host(q.w4a8(xd, wq, s, zq, wsp))
    assert np.array_equal(y.view(np.uint16), yp.view(np.uint16))
    q_ref, s_ref = ref.quantize_activations_int8(x)
    h, l = ref.split_activations_int8(q_ref)
    w = host(ws)
    mk = (M * K + 15) // 16 * 16
    assert np.array_equal(w[:M * K].reshape(M, K), _E4M3[16 * h + 128])
    assert np.array_equal(w[mk:mk + M * K].reshape(M, K), _E4M3[l + 128])
    assert np.array_equal(w[2 * mk:2 * mk + 4 * M].view(np.float32).view(np.uint32), s_ref.view(np.uint32))
    rows = np.arange(N) if N <= 4096 else np.arange(0, N, 7)
    y_ref, A = ref.gemv_w4a8_split(x, c["codes"], c["scales"], c["zeros"], rows=rows)
    assert_within(y[:, rows], y_ref, A, f"w4a8 split M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", SPLIT_SHAPES)
def test_w4a8_asym_matches_oracle_and_quantizes_exactly(M, N, K):
    say("w4a8 asym", M, N, K)
    t = torch()
    c = synth.uniform_case(N + K + 3 * M, M, N, K, 4)
    x = c["x"].copy()
    if M >= 3:
        x[1] = 0                                              # a zero row
        x[2] = np.abs(x[2]) + np.float16(0.5)                 # an all-positive row
        x[2, :2] = [np.float16(60000.0), np.float16(0.25)]    # with an extreme value
    ws = t.zeros(q.w4a8_asym_workspace_bytes(M, K), dtype=t.uint8, device="cuda")
    y = host(q.w4a8_asym(dev(x), *_packed(c), ws))
    xq_ref, sx_ref, zx_ref = ref.quantize_activations_asym8(x)
    w = host(ws)
    mk = (M * K + 15) // 16 * 16
    assert np.array_equal(w[:M * K].view(np.int8).reshape(M, K), xq_ref)
    assert np.array_equal(w[mk:mk + 4 * M].view(np.uint32), sx_ref.view(np.uint32))
    assert np.array_equal(w[mk + 64:mk + 64 + 4 * M].view(np.int32), zx_ref)
    G = K // 128
    sums = w[mk + 128:mk + 128 + 64 * G].view(np.int32).reshape(G, 16)[:, :M].T
    assert np.array_equal(sums, xq_ref.astype(np.int64).reshape(M, G, 128).sum(axis=2))
    rows = np.arange(N) if N <= 4096 else np.arange(0, N, 7)
    y_ref, A = ref.gemv_w4a8_asym(x, c["codes"], c["scales"], c["zeros"], rows=rows)
    assert_within(y[:, rows], y_ref, A, f"w4a8 asym M={M} N={N} K={K}")


@pytest.mark.parametrize("tr", [1, 2])
@pytest.mark.parametrize("M,N,K", [(16, 300, 2048), (6, 8200, 1024)])
def test_w4a8_asym_tile_rows_and_waves(tr, M, N, K, monkeypatch):
    monkeypatch.setenv("QGEMV_W4A8_TR", str(tr))
    for wk in (1, 3, 16):
        monkeypatch.setenv("QGEMV_W4A8_WK", str(wk))
        say("w4a8 asym tr/wk", tr, wk, M, N, K)
        t = torch()
        c = synth.uniform_case(13 * tr + wk + N, M, N, K, 4)
        ws = t.zeros(q.w4a8_asym_workspace_bytes(M, K), dtype=t.uint8, device="cuda")
        y = host(q.w4a8_asym(dev(c["x"]), *_packed(c), ws))
        y_ref, A = ref.gemv_w4a8_asym(c["x"], c["codes"], c["scales"], c["zeros"])
        assert_within(y, y_ref, A, f"w4a8 asym tr={tr} wk={wk} M={M} N={N} K={K}")


def test_w4a8_split_and_asym_degenerate_codes():
    """q == z: every strategy gives exactly 0."""
    t = torch()
    M, N, K = 16, 256, 1024
    c = synth.uniform_case(77, M, N, K, 4)
    c["codes"] = synth.degenerate_codes(78, c["zeros"], 4)
    args = (dev(c["x"]), *_packed(c))
    for fn, wsb in ((q.w4a8_split, q.w4a8_split_workspace_bytes), (q.w4a8_asym, q.w4a8_asym_workspace_bytes)):
        say("w4a8 q==z", fn.__name__)
        y = host(fn(*args, t.zeros(wsb(M, K), dtype=t.uint8, device="cuda")))
        assert np.all(y.astype(np.float64) == 0.0), fn.__name__
