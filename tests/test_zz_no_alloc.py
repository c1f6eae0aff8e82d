"""qgemv_w4a8_noalloc (the entry point that allocates nothing) against
qgemv_w4a8 with a caller workspace: the same kernels, so the same bits, on
two calls in a row (the second smaller, so it reuses the scratch the first
left), and against the float64 oracle's W4A8 definition."""
import ctypes

import numpy as np
import pytest

import synth
from oracle import reference as ref
from tests.gpu_util import assert_within, dev, host, say, torch

pytestmark = pytest.mark.gpu

q = pytest.importorskip("gemm_unpack_bit_amd")


def _case(seed, M, N, K):
    c = synth.uniform_case(seed, M, N, K, 4)
    t = dict(x=dev(c["x"]), wq=q.pack(dev(c["codes"]), 4), s=dev(c["scales"]), z=q.pack_zeros(dev(c["zeros"]), 4))
    return c, t


def _with_ws(t, M, K):
    tt = torch()
    ws = tt.zeros(q.w4a8_workspace_bytes(M, K), dtype=tt.uint8, device="cuda")
    return host(q.w4a8(t["x"], t["wq"], t["s"], t["z"], ws))


def test_noalloc_matches_workspace_call_twice_in_a_row():
    tt = torch()
    shapes = [(16, 4096, 14336, 71), (3, 1000, 2176, 72)]  # second call smaller
    for M, N, K, seed in shapes:
        say("w4a8 noalloc", M, N, K)
        c, t = _case(seed, M, N, K)
        y_ws = _with_ws(t, M, K)
        y = tt.full((M, N), float("nan"), dtype=tt.float16, device="cuda")
        q.w4a8_noalloc(t["x"], t["wq"], t["s"], t["z"], out=y)
        y = host(y)
        assert np.array_equal(y.view(np.uint16), y_ws.view(np.uint16)), (M, N, K)
        rows = np.arange(0, N, 7)
        y_ref, A = ref.gemv_w4a8(c["x"], c["codes"], c["scales"], c["zeros"], rows=rows)
        assert_within(y[:, rows], y_ref, A, f"w4a8 noalloc M={M} N={N} K={K}")


def test_noalloc_largest_size_and_rejection():
    M, N, K = 16, 256, q.W4A8_NOALLOC_MAX_MK // 16
    say("w4a8 noalloc max", M, N, K)
    c, t = _case(73, M, N, K)
    y = host(q.w4a8_noalloc(t["x"], t["wq"], t["s"], t["z"]))
    assert np.array_equal(y.view(np.uint16), _with_ws(t, M, K).view(np.uint16))
    # one group more than the scratch holds: rejected before any launch
    tt = torch()
    x = tt.zeros((16, K + 128), dtype=tt.float16, device="cuda")
    wq = tt.zeros(q.packed_words(4, N, K + 128), dtype=tt.int32, device="cuda")
    s = tt.zeros((N, (K + 128) // 128), dtype=tt.float16, device="cuda")
    z = q.pack_zeros(tt.zeros((N, (K + 128) // 128), dtype=tt.uint8, device="cuda"), 4)
    with pytest.raises(q.QgemvError) as e:
        q.w4a8_noalloc(x, wq, s, z)
    assert e.value.status == q.ERR_WORKSPACE
