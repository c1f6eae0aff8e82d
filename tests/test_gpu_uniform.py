"""GPU parity of the uniform W2/W4/W8 A16 path against the float64 oracle.

Element-by-element checks use |y - y_ref| <= 2e-3 * A + 1e-6 (A = sum |x w|);
packing and the exact special cases are checked bit for bit.
"""
import functools
import os

import numpy as np
import pytest

import synth
from oracle import formats, reference as ref
from tests.gpu_util import assert_within, dev, host, sample_rows, say, torch, uniform_weights

pytestmark = pytest.mark.gpu

q = pytest.importorskip("gemm_unpack_bit_amd")
PATHS = [q.PATH_AUTO, q.PATH_VALU, q.PATH_MFMA]


# ----------------------------------------------------------------------------
# packing
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("R,C", [(1, 8), (3, 37), (16, 256), (33, 1000)])
def test_plain_pack_bit_exact_against_oracle(bits, R, C):
    say("pack plain", bits, R, C)
    codes = synth.codes(R * 1000 + C, 2, R * C, bits).reshape(R, C)
    packed = q.pack(dev(codes), bits, q.LAYOUT_PLAIN)
    assert np.array_equal(host(packed).view(np.uint32), formats.pack_plain(codes, bits))
    assert np.array_equal(host(q.unpack(packed, bits, R, C, q.LAYOUT_PLAIN)), codes)


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("R,C", [(1, 128), (16, 256), (33, 384), (100, 1024)])
def test_device_pack_bit_exact_against_oracle(bits, R, C):
    say("pack device", bits, R, C)
    codes = synth.codes(R * 1000 + C, 2, R * C, bits).reshape(R, C)
    packed = q.pack(dev(codes), bits)
    assert np.array_equal(host(packed).view(np.uint32), formats.pack_tiles(codes, bits))
    assert np.array_equal(host(q.unpack(packed, bits, R, C)), codes)


def test_pack_rejects_out_of_range_code():
    say("pack bad code")
    codes = np.zeros((2, 64), dtype=np.uint8)
    codes[1, 5] = 16
    codes = np.zeros((2, 128), dtype=np.uint8)
    codes[1, 5] = 16
    with pytest.raises(q.QgemvError) as e:
        q.pack(dev(codes), 4)
    assert e.value.status == q.ERR_VALUE
    # the flag is cleared for the next call
    codes[1, 5] = 15
    q.pack(dev(codes), 4)


# ----------------------------------------------------------------------------
# small and ragged shapes: every element against the oracle
# ----------------------------------------------------------------------------
SMALL = [(1, 128), (7, 256), (100, 384), (128, 1024), (300, 2176), (67, 4096)]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("N,K", SMALL)
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 16])
def test_uniform_small_shapes(path, bits, N, K, M):
    say("uniform", path, bits, N, K, M)
    c = synth.uniform_case(N * 7 + K + bits, M, N, K, bits)
    wq = q.pack(dev(c["codes"]), bits)
    zq = q.pack_zeros(dev(c["zeros"]), bits)
    y = q.uniform(dev(c["x"]), wq, dev(c["scales"]), zq, bits, path)
    y_ref, A = ref.gemv_uniform(c["x"], c["codes"], c["scales"], c["zeros"])
    assert_within(host(y), y_ref, A, f"W{bits} M={M} N={N} K={K} path={path}")


# ----------------------------------------------------------------------------
# every launch shape the kernel accepts (forced through QGEMV_TILE_CFG), on a
# ragged shape: whole and partial chunks, tile-rows past N, K/128 odd and even
# ----------------------------------------------------------------------------
LAUNCH_CASES = [(q.PATH_VALU, 1), (q.PATH_VALU, 2), (q.PATH_MFMA, 5)]


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("N,K", [(300, 2176), (200, 2048)])
@pytest.mark.parametrize("path,M", LAUNCH_CASES)
def test_every_launch_shape(monkeypatch, bits, N, K, path, M):
    say("launch shapes", bits, N, K, path, M)
    c = synth.uniform_case(N + K + bits, M, N, K, bits)
    wq = q.pack(dev(c["codes"]), bits)
    zq = q.pack_zeros(dev(c["zeros"]), bits)
    x, s = dev(c["x"]), dev(c["scales"])
    y_ref, A = ref.gemv_uniform(c["x"], c["codes"], c["scales"], c["zeros"])
    ran = []
    for tpw in (1, 2, 4, 8):
        for wk in (1, 4, 16):
            for mt in ((1, 2) if path == q.PATH_VALU else (1,)):
                for v in range(6):
                    cfg = f"{tpw},{wk},{mt},{v}"
                    monkeypatch.setenv("QGEMV_TILE_CFG", cfg)
                    try:
                        y = q.uniform(x, wq, s, zq, bits, path)
                    except q.QgemvError:
                        continue  # a shape this kernel does not take
                    assert_within(host(y), y_ref, A, f"W{bits} M={M} N={N} K={K} path={path} cfg={cfg}")
                    ran.append(cfg)
    assert len(ran) >= 12, ran
    if path == q.PATH_VALU:
        # the deep chunk rings (one tile-row, 4 or 8 one-group chunks in flight)
        assert any(r.startswith("1,") and r.endswith(",4") for r in ran), ran


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("N,K,cfg", [(28672, 4096, None), (4096, 4096, None), (300, 2048, "1,4,1,4"),
                                     (1000, 4096, "1,8,2,4"), (260, 2048, "1,2,1,5"), (10240, 8192, None),
                                     (1000, 4096, "1,8,1,3"), (300, 2048, "1,4,2,3")])
def test_whole_ring_rounds_kernel_equals_general(monkeypatch, bits, N, K, cfg):
    """Where K/128 fills whole rounds of a one-tile-row chunk ring, the
    kernel without the past-the-last-chunk selects runs
    (QGEMV_FULL_ROUNDS=1, the default); it must give the general kernel's y
    bit for bit (8B gate+up and o and 70B q as picked, and forced shapes:
    the 4- and 8-deep rings and the two-stage loop, one and two batch
    rows), inside the oracle's bound on sampled rows."""
    if bits == 8 and cfg and cfg.endswith(",5"):
        pytest.skip("the 8-deep ring holds 8-bit stages only by spilling: no such kernel")
    M = 2 if cfg and cfg.split(",")[2] == "2" else 1
    c = synth.uniform_case(900 + N + bits, M, N, K, bits)
    wq, zq, s, x = q.pack(dev(c["codes"]), bits), q.pack_zeros(dev(c["zeros"]), bits), dev(c["scales"]), dev(c["x"])
    if cfg:
        monkeypatch.setenv("QGEMV_TILE_CFG", cfg)
    ys = {}
    for full in ("0", "1"):
        say("full rounds", full, bits, N, K, cfg)
        monkeypatch.setenv("QGEMV_FULL_ROUNDS", full)
        ys[full] = host(q.uniform(x, wq, s, zq, bits, q.PATH_VALU))
    assert np.array_equal(ys["0"].view(np.uint16), ys["1"].view(np.uint16))
    rows = sample_rows(N)
    y_ref, A = ref.gemv_uniform(c["x"], c["codes"], c["scales"], c["zeros"], rows=rows)
    assert_within(ys["1"][:, rows], y_ref, A, f"full rounds W{bits} N={N} K={K} cfg={cfg}")


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("M", [2, 5, 8, 13, 16])
def test_activation_ring_launch_shapes(monkeypatch, bits, M):
    """Matrix-core engine with the activations not staged whole: each wave
    streams its chunks' activation blocks through a two-slot LDS ring (on and
    off), with staged or per-lane quant params, several tile-rows and wave
    counts; a ragged N, an odd K/128 and batch rows that are not a multiple
    of 4."""
    N, K = 300, 2176
    say("activation ring", bits, M, N, K)
    c = synth.uniform_case(N + K + bits + M, M, N, K, bits)
    wq = q.pack(dev(c["codes"]), bits)
    zq = q.pack_zeros(dev(c["zeros"]), bits)
    x, s = dev(c["x"]), dev(c["scales"])
    y_ref, A = ref.gemv_uniform(c["x"], c["codes"], c["scales"], c["zeros"])
    monkeypatch.setenv("QGEMV_XLDS_MAX", "0")  # activations never staged whole
    for xd in ("2", "0"):  # the ring forced on, and off
        monkeypatch.setenv("QGEMV_XDMA", xd)
        for plds in ("1", "0"):
            monkeypatch.setenv("QGEMV_PLDS", plds)
            for tpw in (2, 4):
                for wk in (1, 4, 16):
                    cfg = f"{tpw},{wk},1,3"
                    monkeypatch.setenv("QGEMV_TILE_CFG", cfg)
                    y = host(q.uniform(x, wq, s, zq, bits, q.PATH_MFMA))
                    assert_within(y, y_ref, A, f"W{bits} M={M} cfg={cfg} xd={xd} plds={plds}")


# ----------------------------------------------------------------------------
# exact special cases
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("bits", [2, 4, 8])
def test_one_hot_x_is_bit_exact(path, bits):
    """x = e_k gives y[n] = fp16(s * (q - z)) for every (q, z) pair."""
    say("one-hot", path, bits)
    L = 1 << bits
    qs, zs = np.meshgrid(np.arange(L), np.arange(L), indexing="ij")
    N = L * L
    K = 512
    for k in (0, 129, 511):
        codes = synth.codes(k, 3, N * K, bits).reshape(N, K)
        codes[:, k] = qs.reshape(-1)
        zeros = synth.codes(k, 4, N * 4, bits).reshape(N, 4)
        zeros[:, k // 128] = zs.reshape(-1)
        scales = synth.f16(synth.uniform(k, 5, N * 4, 0.001, 0.02)).reshape(N, 4)
        x = np.zeros((1, K), dtype=np.float16)
        x[0, k] = 1.0
        y = q.uniform(dev(x), q.pack(dev(codes), bits), dev(scales), q.pack_zeros(dev(zeros), bits), bits, path)
        want = (scales[:, k // 128].astype(np.float64) * (qs.reshape(-1) - zs.reshape(-1))).astype(np.float16)
        assert np.array_equal(host(y)[0].view(np.uint16), want.view(np.uint16))


DEGENERATE_SHAPES = [(96, 1024), (300, 2176), (28672, 4096), (4096, 14336)]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("N,K", DEGENERATE_SHAPES)
def test_codes_equal_zero_points_give_exact_zero(path, bits, N, K):
    """q == z everywhere: y = 0 exactly (A = 0, so the bound is 1e-6), on every
    engine and batch size, in the launch shapes the bench uses (the 8B gate+up
    and down layers) and on small and ragged ones."""
    c = synth.uniform_case(40 + bits + N, 16, N, K, bits)
    codes = synth.degenerate_codes(41, c["zeros"], bits)
    wq, zq, s = q.pack(dev(codes), bits), q.pack_zeros(dev(c["zeros"]), bits), dev(c["scales"])
    for M in (1, 2, 4, 16):
        say("q==z", path, bits, N, K, M)
        y = host(q.uniform(dev(c["x"][:M]), wq, s, zq, bits, path))
        assert np.all(y.astype(np.float64) == 0.0), f"W{bits} N={N} K={K} M={M} path={path}"


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("N,K", DEGENERATE_SHAPES)
def test_near_degenerate_codes_within_tolerance(path, bits, N, K):
    """One code per (row, group) one step from z, the rest equal to z: A is
    small (a single weight per group), so a residue that scales with the
    activations rather than with A fails here."""
    c = synth.uniform_case(50 + bits + N, 16, N, K, bits)
    codes = synth.degenerate_codes(51, c["zeros"], bits, near=True)
    wq, zq, s = q.pack(dev(codes), bits), q.pack_zeros(dev(c["zeros"]), bits), dev(c["scales"])
    y_ref, A = ref.gemv_uniform(c["x"], codes, c["scales"], c["zeros"])
    for M in (1, 2, 4, 16):
        say("near q==z", path, bits, N, K, M)
        y = host(q.uniform(dev(c["x"][:M]), wq, s, zq, bits, path))
        assert_within(y, y_ref[:M], A[:M], f"near-degenerate W{bits} N={N} K={K} M={M} path={path}")


def test_subnormal_and_large_activations():
    say("subnormal/large x")
    c = synth.uniform_case(50, 2, 64, 512, 4)
    x = c["x"].astype(np.float64)
    x[0] = x[0] * 2.0 ** -17          # mostly subnormal fp16 values
    x[1] = x[1] * 3000.0              # large but finite
    c["x"] = x.astype(np.float16)
    y = q.uniform(dev(c["x"]), q.pack(dev(c["codes"]), 4), dev(c["scales"]), q.pack_zeros(dev(c["zeros"]), 4), 4)
    y_ref, A = ref.gemv_uniform(c["x"], c["codes"], c["scales"], c["zeros"])
    assert_within(host(y), y_ref, A, "subnormal/large x")


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_output_fully_written_and_deterministic(bits):
    say("poison/determinism", bits)
    t = torch()
    c = synth.uniform_case(60 + bits, 3, 1000, 2048, bits)
    args = (dev(c["x"]), q.pack(dev(c["codes"]), bits), dev(c["scales"]), q.pack_zeros(dev(c["zeros"]), bits))
    y1 = t.full((3, 1000), float("nan"), dtype=t.float16, device="cuda")
    q.uniform(*args, bits, out=y1)
    y2 = t.full((3, 1000), float("nan"), dtype=t.float16, device="cuda")
    q.uniform(*args, bits, out=y2)
    a, b = host(y1), host(y2)
    assert not np.isnan(a.astype(np.float32)).any()
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def test_bad_arguments_raise():
    say("bad args")
    t = torch()
    x = t.zeros((1, 256), dtype=t.float16, device="cuda")
    wq = t.zeros((16 * 32,), dtype=t.int32, device="cuda")
    s = t.zeros((8, 2), dtype=t.float16, device="cuda")
    z = t.zeros((8, 1), dtype=t.int32, device="cuda")
    with pytest.raises(q.QgemvError) as e:
        q.uniform(x[:, :200].contiguous(), wq, s, z, 4)
    assert e.value.status == q.ERR_SHAPE
    with pytest.raises(q.QgemvError):
        q.uniform(x, wq, s, z, 3)


# ----------------------------------------------------------------------------
# full workload sizes, every row against the oracle, in the launch
# configurations the bench uses
# ----------------------------------------------------------------------------
LLAMA8B = list(synth.LLAMA3_8B_LAYERS.items())
LLAMA70B = list(synth.LLAMA_70B_LAYERS.items())


@functools.lru_cache(maxsize=1)
def _oracle_all_rows(seed, N, K, bits):
    """float64 result and tolerance scale of every row for the 16 activation
    rows of the cached case (row m of y depends on row m of x only)."""
    c, _, _, _ = uniform_weights(seed, N, K, bits)
    return ref.gemv_uniform(c["x"], c["codes"], c["scales"], c["zeros"])


def _full_check(seed, name, N, K, bits, Ms, paths):
    c, wq, s, zq = uniform_weights(seed, N, K, bits)
    y_ref, A = _oracle_all_rows(seed, N, K, bits)
    for M in Ms:
        for path in paths:
            say("full", name, N, K, bits, M, "path", path)
            y = host(q.uniform(dev(c["x"][:M]), wq, s, zq, bits, path))
            assert_within(y, y_ref[:M], A[:M], f"{name} W{bits} M={M} path={path}")


@pytest.mark.parametrize("bits", [4, 8, 2])
@pytest.mark.parametrize("idx", range(4))
def test_llama8b_layers_all_rows(bits, idx):
    name, (N, K) = LLAMA8B[idx]
    _full_check(synth.seed_for(1, idx), name, N, K, bits, (1, 2, 4, 16), paths=(q.PATH_AUTO, q.PATH_VALU, q.PATH_MFMA))


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("idx", range(4))
def test_llama70b_layers_all_rows(bits, idx):
    name, (N, K) = LLAMA70B[idx]
    _full_check(synth.seed_for(2, idx), name, N, K, bits, (1, 2, 4, 8, 16), paths=(q.PATH_VALU, q.PATH_MFMA))
