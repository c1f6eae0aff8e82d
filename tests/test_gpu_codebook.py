"""GPU parity of the codebook (Psumbook) variant against the float64 oracle:
m = 1 codebook of 256 centroids x 4 dims, 8-bit codes, one scale per 128 k."""
import numpy as np
import pytest

import synth
from oracle import formats, reference as ref
from tests.gpu_util import assert_within, dev, host, sample_rows, say, torch

pytestmark = pytest.mark.gpu

q = pytest.importorskip("gemm_unpack_bit_amd")


def _upload(c):
    return q.pack(dev(c["codes"]), 8, q.LAYOUT_ROWS64), dev(c["codebook"]), dev(c["scales"])


@pytest.mark.parametrize("R,C", [(1, 16), (64, 128), (70, 40), (200, 2048)])
def test_rows64_pack_bit_exact_against_oracle(R, C):
    say("pack rows64", R, C)
    codes = synth.codes(R + C, 2, R * C, 8).reshape(R, C)
    packed = q.pack(dev(codes), 8, q.LAYOUT_ROWS64)
    assert np.array_equal(host(packed).view(np.uint8), formats.pack_codebook_tiles(codes))
    assert np.array_equal(host(q.unpack(packed, 8, R, C, q.LAYOUT_ROWS64)), codes)


def _ws(M, N, K):
    t = torch()
    n = q.codebook_workspace_bytes(M, N, K)
    return t.zeros(max(n, 4), dtype=t.uint8, device="cuda") if n else None


@pytest.mark.parametrize("use_ws", [False, True])
@pytest.mark.parametrize("N,K", [(16, 512), (100, 1024), (300, 2048), (70, 1536), (1000, 4096)])
@pytest.mark.parametrize("M", [1, 2, 4, 16])
def test_codebook_small_shapes(use_ws, N, K, M):
    say("codebook", use_ws, N, K, M)
    c = synth.codebook_case(N * 5 + K, M, N, K)
    codes, cb, s = _upload(c)
    y = host(q.codebook(dev(c["x"]), codes, cb, s, ws=_ws(M, N, K) if use_ws else None))
    y_ref, A = ref.gemv_codebook(c["x"], c["codes"], c["codebook"], c["scales"])
    assert_within(y, y_ref, A, f"codebook M={M} N={N} K={K} ws={use_ws}")


@pytest.mark.parametrize("M,N,K", [(1, 300, 3584), (3, 200, 2048), (16, 70, 1536), (2, 1000, 512)])
def test_codebook_every_launch_shape(monkeypatch, M, N, K):
    """Both kernels at every workgroup size (1..16 waves, so every split of
    the build): the stationary one with one, two and four pairs per workgroup,
    Psumbook entries of 1, 2 and 4 batch rows, and
    1 to all row slices, the sequential one with K splits up to one 256-k pair
    per range; each against the oracle."""
    say("codebook launch shapes", M, N, K)
    c = synth.codebook_case(N + K + M, M, N, K)
    codes, cb, s = _upload(c)
    x = dev(c["x"])
    y_ref, A = ref.gemv_codebook(c["x"], c["codes"], c["codebook"], c["scales"])
    ws = torch().zeros(K // 256 * M * N * 4, dtype=torch().uint8, device="cuda")
    NB = (N + 63) // 64
    cfgs = [f"0,{wk},{ks}" for wk in (1, 2, 4, 8, 16) for ks in sorted({1, 2, 3, K // 256})]
    cfgs += [f"1,{wk},{pp},{r}" for wk in (1, 2, 4, 8, 16) for pp in (1, 2, 4) for r in sorted({1, 2, 3, NB})
             if (K // 256) % pp == 0 and not (pp == 4 and wk > 8)]
    # batched Psumbook entries: 2 or 4 batch rows per lookup
    cfgs += [f"1,{wk},{pp},{r},{mb}" for wk in (1, 2, 4, 8) for mb in (2, 4) for pp in (1, 2) for r in sorted({1, 3, NB})
             if (K // 256) % pp == 0 and pp * mb <= 4]
    for cfg in cfgs:
        monkeypatch.setenv("QGEMV_CODEBOOK_CFG", cfg)
        y = host(q.codebook(x, codes, cb, s, ws=ws))
        assert_within(y, y_ref, A, f"codebook M={M} N={N} K={K} cfg={cfg}")


def test_codebook_one_hot_is_exact():
    """x = e_k: y[n] = fp16(s * C[code][k % 4]) exactly."""
    say("codebook one-hot")
    N, K = 64, 1024
    c = synth.codebook_case(3, 1, N, K)
    codes, cb, s = _upload(c)
    w = ref.dequant_codebook(c["codes"], c["codebook"], c["scales"])
    for k in (0, 1, 2, 3, 127, 128, 515, 1023):
        x = np.zeros((1, K), dtype=np.float16)
        x[0, k] = 1.0
        y = host(q.codebook(dev(x), codes, cb, s))
        assert np.array_equal(y[0].view(np.uint16), synth.f16(w[:, k]).view(np.uint16)), k


def test_codebook_deterministic_and_workspace_reusable():
    say("codebook determinism")
    M, N, K = 1, 8192, 8192
    c = synth.codebook_case(7, M, N, K)
    codes, cb, s = _upload(c)
    x = dev(c["x"])
    ws = _ws(M, N, K)
    y1 = host(q.codebook(x, codes, cb, s, ws=ws))
    y2 = host(q.codebook(x, codes, cb, s, ws=ws))
    assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))
    rows = sample_rows(N)
    y_ref, A = ref.gemv_codebook(c["x"], c["codes"], c["codebook"], c["scales"], rows=rows)
    assert_within(y1[:, rows], y_ref, A, "codebook 8192 ws reuse")


@pytest.mark.parametrize("idx", range(4))
def test_codebook_70b_layers(idx):
    name, (N, K) = list(synth.LLAMA_70B_LAYERS.items())[idx]
    say("codebook full", name, N, K)
    c = synth.codebook_case(synth.seed_for(5, idx), 4, N, K)
    codes, cb, s = _upload(c)
    rows = sample_rows(N)
    for M in (1, 4):
        x = c["x"][:M]
        y = host(q.codebook(dev(x), codes, cb, s, ws=_ws(M, N, K)))
        y_ref, A = ref.gemv_codebook(x, c["codes"], c["codebook"], c["scales"], rows=rows)
        assert_within(y[:, rows], y_ref, A, f"codebook {name} M={M}")
        assert np.isfinite(y.astype(np.float32)).all()


def test_one_workspace_serves_several_shapes():
    """A single zero-filled workspace, passed with the same size every time,
    serves layers of different shapes called in any order."""
    say("codebook shared workspace")
    t = torch()
    shapes = [(1, 8192, 8192), (1, 10240, 8192), (4, 8192, 8192)]
    size = max(q.codebook_workspace_bytes(M, N, K) for M, N, K in shapes)
    ws = t.zeros(size, dtype=t.uint8, device="cuda")
    cases = []
    for i, (M, N, K) in enumerate(shapes):
        c = synth.codebook_case(40 + i, M, N, K)
        cases.append((c, _upload(c), sample_rows(N)))
    for rnd in range(2):
        for (M, N, K), (c, (codes, cb, s), rows) in zip(shapes, cases):
            y = host(q.codebook(dev(c["x"]), codes, cb, s, ws=ws))
            y_ref, A = ref.gemv_codebook(c["x"], c["codes"], c["codebook"], c["scales"], rows=rows)
            assert_within(y[:, rows], y_ref, A, f"shared ws round {rnd} M={M} N={N}")
