"""GPU parity of the LUT4 (NF4-style) variant against the float64 oracle.

w[n, k] = lut[q[n, k]] * absmax[n, k / 64]; element checks use
|y - y_ref| <= 2e-3 * A + 1e-6, one-hot activations are checked bit for bit.
"""
import numpy as np
import pytest

import synth
from oracle import reference as ref
from tests.gpu_util import assert_within, dev, host, sample_rows, say, torch

pytestmark = pytest.mark.gpu

q = pytest.importorskip("gemm_unpack_bit_amd")

SMALL = [(1, 128), (7, 256), (100, 384), (128, 1024), (300, 2176), (67, 4096), (900, 1152)]


def _upload(c):
    return q.pack(dev(c["codes"]), 4), dev(c["absmax"]), dev(c["lut"])


@pytest.mark.parametrize("N,K", SMALL)
@pytest.mark.parametrize("M", [1, 2, 3, 16])
def test_lut4_small_shapes(N, K, M):
    say("lut4", N, K, M)
    c = synth.lut4_case(N * 11 + K, M, N, K)
    wq, a, lut = _upload(c)
    y = q.lut4(dev(c["x"]), wq, a, lut)
    y_ref, A = ref.gemv_lut4(c["x"], c["codes"], c["absmax"], c["lut"])
    assert_within(host(y), y_ref, A, f"lut4 M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", [(1, 300, 2176), (2, 200, 2048), (3, 64, 512), (16, 40, 1152)])
def test_lut4_every_launch_shape(monkeypatch, M, N, K):
    """Every launch shape: one tile-row per workgroup with 1- and 2-group
    chunks through 2-, 4- and 8-slot rings, two tile-rows with 4-group
    chunks, 1 to 8 waves, one and two staged activation rows."""
    say("lut4 launch shapes", M, N, K)
    c = synth.lut4_case(N + K + M, M, N, K)
    wq, a, lut = _upload(c)
    x = dev(c["x"])
    y_ref, A = ref.gemv_lut4(c["x"], c["codes"], c["absmax"], c["lut"])
    cfgs = [(1, ng, wk, mt, d) for ng in (1, 2) for wk in (1, 3, 8) for mt in (1, 2) for d in (2, 4, 8)
            if not (ng == 2 and d == 8)]
    cfgs += [(2, 4, wk, mt, 2) for wk in (1, 3, 8) for mt in (1, 2)]
    for bs in ("2", "0"):  # one tile-row of one-group chunks: block scales staged in LDS or loaded per lane
        monkeypatch.setenv("QGEMV_LUT4_BS", bs)
        for cfg in cfgs:
            monkeypatch.setenv("QGEMV_LUT4_CFG", ",".join(map(str, cfg)))
            y = host(q.lut4(x, wq, a, lut))
            assert_within(y, y_ref, A, f"lut4 M={M} N={N} K={K} cfg={cfg} bs={bs}")


@pytest.mark.parametrize("M,N,K", [(1, 33000, 384), (1, 40008, 1024), (2, 20000, 512)])
def test_lut4_many_row_groups_every_row(M, N, K):
    """More row groups than resident workgroups, so each workgroup walks
    several and stages the next group's block scales while it computes the
    current one; a ragged last tile-row; every row checked."""
    say("lut4 many row groups", M, N, K)
    c = synth.lut4_case(N + K + 3 * M, M, N, K)
    wq, a, lut = _upload(c)
    y = host(q.lut4(dev(c["x"]), wq, a, lut))
    y_ref, A = ref.gemv_lut4(c["x"], c["codes"], c["absmax"], c["lut"])
    assert_within(y, y_ref, A, f"lut4 M={M} N={N} K={K}")


def test_lut4_one_hot_is_exact():
    """x = e_k: y[n] = fp16(lut[q] * a) exactly (a single product, rounded once)."""
    say("lut4 one-hot")
    N, K = 48, 512
    c = synth.lut4_case(7, 1, N, K)
    wq, a, lut = _upload(c)
    for k in (0, 1, 63, 64, 130, 511):
        x = np.zeros((1, K), dtype=np.float16)
        x[0, k] = 1.0
        y = host(q.lut4(dev(x), wq, a, lut))
        want = synth.f16(ref.dequant_lut4(c["codes"], c["absmax"], c["lut"])[:, k])
        assert np.array_equal(y[0].view(np.uint16), want.view(np.uint16)), k


def test_lut4_arbitrary_table_and_zero_scale():
    """The table is an input: a permuted, signed, unevenly spaced table works;
    rows whose scales are zero give exactly 0."""
    say("lut4 table")
    N, K = 70, 768
    c = synth.lut4_case(9, 2, N, K)
    c["lut"] = synth.f16(np.array([3.5, -0.25, 7, 0, -6, 1.125, 2, -2, 0.5, 9, -9, 4, -1.5, 6, -3, 1]))
    c["absmax"][5] = 0
    wq, a, lut = _upload(c)
    y = host(q.lut4(dev(c["x"]), wq, a, lut))
    y_ref, A = ref.gemv_lut4(c["x"], c["codes"], c["absmax"], c["lut"])
    assert_within(y, y_ref, A, "lut4 arbitrary table")
    assert np.all(y[:, 5] == 0)


def test_lut4_deterministic():
    say("lut4 determinism")
    N, K = 4096, 4096
    c = synth.lut4_case(5, 1, N, K)
    wq, a, lut = _upload(c)
    x = dev(c["x"])
    y1 = host(q.lut4(x, wq, a, lut))
    y2 = host(q.lut4(x, wq, a, lut))
    assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))


@pytest.mark.parametrize("idx", range(4))
def test_lut4_llama8b_layers(idx):
    name, (N, K) = list(synth.LLAMA3_8B_LAYERS.items())[idx]
    say("lut4 full", name, N, K)
    c = synth.lut4_case(synth.seed_for(1, 16 + idx), 16, N, K)
    wq, a, lut = _upload(c)
    rows = sample_rows(N)
    for M in (1, 4):
        x = c["x"][:M]
        y = host(q.lut4(dev(x), wq, a, lut))
        y_ref, A = ref.gemv_lut4(x, c["codes"], c["absmax"], c["lut"], rows=rows)
        assert_within(y[:, rows], y_ref, A, f"lut4 {name} M={M}")
        assert np.isfinite(y.astype(np.float32)).all()


def test_lut4_bad_arguments_raise():
    say("lut4 bad args")
    t = torch()
    x = t.zeros((1, 256), dtype=t.float16, device="cuda")
    wq = t.zeros((16 * 32,), dtype=t.int32, device="cuda")
    a = t.zeros((8, 4), dtype=t.float16, device="cuda")
    lut = t.zeros((16,), dtype=t.float16, device="cuda")
    with pytest.raises(q.QgemvError) as e:
        q.lut4(x[:, :192].contiguous(), wq, a, lut)
    assert e.value.status == q.ERR_SHAPE
    with pytest.raises(ValueError):
        q.lut4(x, wq, a, lut[:8])
