"""GPU parity of the general codebook GEMV (m additive codebooks, vector length
v, scale group g) against the float64 oracle."""
import numpy as np
import pytest

import synth
from oracle import reference as ref
from tests.gpu_util import assert_within, dev, host, sample_rows, say, torch

pytestmark = pytest.mark.gpu

q = pytest.importorskip("gemm_unpack_bit_amd")

FORMATS = [(1, 4, 128), (1, 4, 32), (1, 8, 64), (2, 8, 128), (1, 16, 128), (2, 16, 64), (3, 16, 32), (4, 16, 32)]


def _run(c, g, ws=True, M=None):
    t = torch()
    ncb, N, KC = c["codes"].shape
    v = c["codebooks"].shape[2]
    x = dev(c["x"])
    M, K = x.shape
    codes = q.pack_codebook_planes(dev(c["codes"]))
    w = None
    if ws:
        nb = q.codebook_gen_workspace_bytes(M, N, K, ncb, v, g)
        w = t.zeros(max(nb, 4) // 4, dtype=t.int32, device="cuda")
    return host(q.codebook_gen(x, codes, dev(c["codebooks"]), dev(c["scales"]), g, ws=w))


@pytest.mark.parametrize("m,v,g", FORMATS)
@pytest.mark.parametrize("M,N,K", [(1, 300, 2048), (3, 200, 1024), (16, 70, 512), (2, 1000, 256)])
def test_codebook_gen_small_shapes(m, v, g, M, N, K):
    say("codebook gen", m, v, g, M, N, K)
    c = synth.codebook_additive_case(N + K + 7 * m + v, M, N, K, m, v, g)
    y = _run(c, g)
    y_ref, A = ref.gemv_codebook_additive(c["x"], c["codes"], c["codebooks"], c["scales"], g)
    assert_within(y, y_ref, A, f"codebook gen m={m} v={v} g={g} M={M} N={N} K={K}")


@pytest.mark.parametrize("m,v,g", [(1, 4, 128), (3, 16, 32)])
def test_codebook_gen_without_workspace(m, v, g):
    """No workspace: one K range per workgroup, same result within the tolerance."""
    N, K, M = 500, 4096, 2
    say("codebook gen no ws", m, v, g)
    c = synth.codebook_additive_case(41 + m, M, N, K, m, v, g)
    y = _run(c, g, ws=False)
    y_ref, A = ref.gemv_codebook_additive(c["x"], c["codes"], c["codebooks"], c["scales"], g)
    assert_within(y, y_ref, A, f"codebook gen no ws m={m} v={v}")


@pytest.mark.parametrize("ks", ["1", "2", "5", "16"])
def test_codebook_gen_every_k_split(ks, monkeypatch):
    N, K, M = 333, 4096, 3
    say("codebook gen ks", ks)
    c = synth.codebook_additive_case(43, M, N, K, 2, 8, 64)
    monkeypatch.setenv("QGEMV_CODEBOOK_GEN_KS", ks)
    t = torch()
    w = t.zeros((16 * M * N), dtype=t.int32, device="cuda")
    y = host(q.codebook_gen(dev(c["x"]), q.pack_codebook_planes(dev(c["codes"])), dev(c["codebooks"]),
                            dev(c["scales"]), 64, ws=w))
    y_ref, A = ref.gemv_codebook_additive(c["x"], c["codes"], c["codebooks"], c["scales"], 64)
    assert_within(y, y_ref, A, f"codebook gen ks={ks}")


def test_codebook_gen_single_codebook_matches_specialized_kernel():
    """m = 1, v = 4, g = 128 is the specialized kernel's format: both agree
    within the tolerance (different summation orders)."""
    N, K, M = 1024, 4096, 1
    say("codebook gen vs specialized")
    c = synth.codebook_additive_case(44, M, N, K, 1, 4, 128)
    y = _run(c, 128)
    t = torch()
    ws = t.zeros(max(q.codebook_workspace_bytes(M, N, K), 4) // 4, dtype=t.int32, device="cuda")
    ys = host(q.codebook(dev(c["x"]), q.pack(dev(c["codes"][0]), 8, q.LAYOUT_ROWS64), dev(c["codebooks"][0]),
                         dev(c["scales"]), ws=ws))
    y_ref, A = ref.gemv_codebook(c["x"], c["codes"][0], c["codebooks"][0], c["scales"])
    assert_within(y, y_ref, A, "gen")
    assert_within(ys, y_ref, A, "specialized")


@pytest.mark.parametrize("m,v,g", [(3, 16, 32), (1, 4, 32)])
def test_codebook_gen_full_size_gate_up(m, v, g):
    N, K, M = 28672, 4096, 1
    say("codebook gen full", m, v, g)
    c = synth.codebook_additive_case(45, M, N, K, m, v, g)
    y = _run(c, g)
    rows = sample_rows(N)
    y_ref, A = ref.gemv_codebook_additive(c["x"], c["codes"], c["codebooks"], c["scales"], g, rows=rows)
    assert_within(y[:, rows], y_ref, A, f"codebook gen full m={m} v={v} g={g}")


@pytest.mark.parametrize("m,v,g", FORMATS)
@pytest.mark.parametrize("wk", ["-1", "-2", "-4"])
def test_codebook_gen_stationary_form(m, v, g, wk, monkeypatch):
    """The stationary form (one K part per 256-k chunk, rows streamed through
    each chunk's Psumbooks) at every workgroup size, on ragged rows."""
    N, K, M = 777, 2048, 2
    say("codebook gen stationary", m, v, g, wk)
    c = synth.codebook_additive_case(47 + m + v, M, N, K, m, v, g)
    monkeypatch.setenv("QGEMV_CODEBOOK_GEN_KS", wk)
    y = _run(c, g)
    y_ref, A = ref.gemv_codebook_additive(c["x"], c["codes"], c["codebooks"], c["scales"], g)
    assert_within(y, y_ref, A, f"codebook gen stationary m={m} v={v} g={g} wk={wk}")
