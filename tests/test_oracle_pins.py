"""Pins for the float64 oracle against exact arithmetic, closed forms,
identities and the facts the pages print (CPU only).

Each pin is chosen so that a plausible slip in the oracle -- a dropped term,
a sign, an off-by-one group index, a transposed operand -- fails at least one
test here; ``test_planted_mistakes_are_caught`` checks exactly that.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import exact, reference as ref


def _tiny_uniform(seed, M, N, K, bits):
    return synth.uniform_case(seed, M, N, K, bits)


# ----------------------------------------------------------------------------
# exact brute force on tiny shapes
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("M,N,K", [(1, 3, 128), (3, 5, 256)])
def test_uniform_matches_exact(bits, M, N, K):
    c = _tiny_uniform(100 + bits, M, N, K, bits)
    y, A = ref.gemv_uniform(c["x"], c["codes"], c["scales"], c["zeros"])
    ye = exact.to_f64(exact.gemv_uniform_exact(c["x"], c["codes"], c["scales"], c["zeros"]))
    assert np.all(np.abs(y - ye) <= 1e-12 * A + 1e-300)
    assert np.all(A > 0)


def test_lut4_matches_exact():
    c = synth.lut4_case(5, 2, 4, 256)
    y, A = ref.gemv_lut4(c["x"], c["codes"], c["absmax"], c["lut"])
    ye = exact.to_f64(exact.gemv_lut4_exact(c["x"], c["codes"], c["absmax"], c["lut"]))
    assert np.all(np.abs(y - ye) <= 1e-12 * A)


def test_codebook_matches_exact():
    c = synth.codebook_case(6, 2, 3, 256)
    y, A = ref.gemv_codebook(c["x"], c["codes"], c["codebook"], c["scales"])
    ye = exact.to_f64(exact.gemv_codebook_exact(c["x"], c["codes"], c["codebook"], c["scales"]))
    assert np.all(np.abs(y - ye) <= 1e-12 * A)


def test_outlier_matches_exact():
    c = synth.outlier_case(8, 2, 6, 256, frac=0.02)
    y, A = ref.gemv_outlier(c["x"], c["codes"], c["scales"], c["zeros"],
                            c["o_rows"], c["o_cols"], c["o_vals"])
    yd = exact.gemv_uniform_exact(c["x"], c["codes"], c["scales"], c["zeros"])
    ys = exact.sparse_exact(c["x"], 6, c["o_rows"], c["o_cols"], c["o_vals"])
    ye = exact.to_f64([[a + b for a, b in zip(r1, r2)] for r1, r2 in zip(yd, ys)])
    assert len(c["o_rows"]) == int(0.02 * 6 * 256)
    assert np.all(np.abs(y - ye) <= 1e-12 * A)


# ----------------------------------------------------------------------------
# closed forms and identities
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("bits", [2, 4, 8])
def test_one_hot_x_gives_single_dequantized_weight(bits):
    """x = e_k  =>  y[n] = s[n, k//128] * (q[n,k] - z[n, k//128]), every (q, z)."""
    L = 1 << bits
    qs, zs = np.meshgrid(np.arange(L), np.arange(L), indexing="ij")
    N = L * L
    K = 256
    k = 131  # second group
    codes = np.zeros((N, K), dtype=np.uint8)
    codes[:, k] = qs.reshape(-1)
    zeros = np.zeros((N, 2), dtype=np.uint8)
    zeros[:, 1] = zs.reshape(-1)
    zeros[:, 0] = (zs.reshape(-1) + 1) % L  # must not leak into the answer
    scales = synth.f16(np.linspace(0.001, 0.02, N * 2)).reshape(N, 2)
    x = np.zeros((1, K), dtype=np.float16)
    x[0, k] = 1.0
    y, A = ref.gemv_uniform(x, codes, scales, zeros)
    want = scales[:, 1].astype(np.float64) * (qs.reshape(-1) - zs.reshape(-1))
    assert np.array_equal(y[0], want)
    assert np.array_equal(A[0], np.abs(want))


def test_all_ones_x_closed_form():
    c = _tiny_uniform(11, 1, 7, 384, 4)
    x = np.ones((1, 384), dtype=np.float16)
    y, _ = ref.gemv_uniform(x, c["codes"], c["scales"], c["zeros"])
    for n in range(7):
        want = 0.0
        for G in range(3):
            qsum = int(c["codes"][n, 128 * G:128 * (G + 1)].astype(np.int64).sum())
            want += float(c["scales"][n, G]) * (qsum - 128 * int(c["zeros"][n, G]))
        assert y[0, n] == pytest.approx(want, rel=1e-14, abs=1e-14)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_codes_equal_zero_points_give_zero(bits):
    c = _tiny_uniform(12, 2, 9, 256, bits)
    codes = np.repeat(c["zeros"], 128, axis=1)
    y, A = ref.gemv_uniform(c["x"], codes, c["scales"], c["zeros"])
    assert np.all(y == 0.0) and np.all(A == 0.0)


def test_unit_scale_zero_offset_is_integer_matvec():
    rng = np.random.default_rng(3)
    N, K, M = 6, 256, 2
    codes = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    xi = rng.integers(-8, 9, size=(M, K))
    x = xi.astype(np.float16)
    y, _ = ref.gemv_uniform(x, codes, np.ones((N, 2), dtype=np.float16), np.zeros((N, 2), dtype=np.uint8))
    want = xi.astype(object) @ codes.astype(object).T
    assert np.array_equal(y.astype(np.int64), np.array(want, dtype=np.int64))


def test_group_identity_matches_direct():
    """QFactory zero-point expansion specialised to one group."""
    c = _tiny_uniform(13, 3, 40, 512, 4)
    y, A = ref.gemv_uniform(c["x"], c["codes"], c["scales"], c["zeros"])
    yi = ref.gemv_uniform_identity(c["x"], c["codes"], c["scales"], c["zeros"])
    sx = np.abs(c["x"].astype(np.float64)).sum(axis=1, keepdims=True)
    assert np.all(np.abs(y - yi) <= 1e-12 * (A + 16 * 0.02 * sx))


def test_zero_point_expansion_page_example(golden_dir):
    with open(os.path.join(golden_dir, "page_facts.json")) as f:
        fx = json.load(f)["zero_point_expansion"]
    A = np.array(fx["A"], dtype=object)
    B = np.array(fx["B"], dtype=object)
    z1, z2 = fx["z1"], fx["z2"]
    K = A.shape[1]
    JA = np.ones(A.shape, dtype=object)
    JB = np.ones(B.shape, dtype=object)
    expanded = A @ B - z1 * (JA @ B) - z2 * (A @ JB) + z1 * z2 * K * np.ones((A.shape[0], B.shape[1]), dtype=object)
    assert expanded.tolist() == fx["product"]
    # and the oracle's dequantized product agrees with it: rows of B^T are weight rows
    codes = np.array(B.T, dtype=np.uint8)          # [N=2, K=3] codes
    x = np.array(A, dtype=np.float16)              # [M=2, K=3] activations; shift x by z1:
    x = (x.astype(np.float64) - z1).astype(np.float16)
    # pad K to one full group of 128 with zero activations and code == zero point
    Kp = 128
    xp = np.zeros((2, Kp), dtype=np.float16); xp[:, :3] = x
    cp = np.full((2, Kp), z2, dtype=np.uint8); cp[:, :3] = codes
    y, _ = ref.gemv_uniform(xp, cp, np.ones((2, 1), dtype=np.float16), np.full((2, 1), z2, dtype=np.uint8))
    assert y.tolist() == fx["product"]


def test_rows_are_independent():
    c = _tiny_uniform(14, 4, 10, 256, 2)
    y, A = ref.gemv_uniform(c["x"], c["codes"], c["scales"], c["zeros"])
    for m in range(4):
        y1, A1 = ref.gemv_uniform(c["x"][m:m + 1], c["codes"], c["scales"], c["zeros"])
        assert np.array_equal(y1[0], y[m]) and np.array_equal(A1[0], A[m])
    ys, As = ref.gemv_uniform(c["x"], c["codes"], c["scales"], c["zeros"], rows=[7, 2])
    assert np.array_equal(ys, y[:, [7, 2]]) and np.array_equal(As, A[:, [7, 2]])


def test_lut4_one_hot_and_reduction_to_uniform():
    c = _tiny_uniform(15, 2, 8, 256, 4)
    z0 = 6
    lut = np.arange(16, dtype=np.float64) - z0
    lut16 = lut.astype(np.float16)
    absmax = np.repeat(c["scales"], 2, axis=1)    # same scale on both 64-blocks
    yl, Al = ref.gemv_lut4(c["x"], c["codes"], absmax, lut16)
    yu, Au = ref.gemv_uniform(c["x"], c["codes"], c["scales"], np.full_like(c["zeros"], z0))
    assert np.allclose(yl, yu, rtol=0, atol=1e-12 * Au.max()) and np.allclose(Al, Au, rtol=1e-14)
    # one-hot x picks LUT[q] * a for the block of k
    lc = synth.lut4_case(16, 1, 16, 128)
    codes = np.arange(16, dtype=np.uint8)[:, None].repeat(128, axis=1)
    x = np.zeros((1, 128), dtype=np.float16); x[0, 70] = 1.0
    y, _ = ref.gemv_lut4(x, codes, lc["absmax"], lc["lut"])
    want = lc["lut"].astype(np.float64) * lc["absmax"][:, 1].astype(np.float64)
    assert np.array_equal(y[0], want)


def test_lut_levels_are_sorted_and_symmetric(golden_dir):
    with open(os.path.join(golden_dir, "page_facts.json")) as f:
        nf4 = json.load(f)["nf4_lut"]
    L = synth.normal_quantile_levels(nf4["levels"]).astype(np.float64)
    assert L.size == nf4["levels"] and L.size * 4 == nf4["shared_bytes_per_block"]  # fp32 LUT fits
    assert np.all(np.diff(L) > 0) and L[-1] == 1.0 and L[0] == -1.0
    assert np.allclose(L, -L[::-1])
    assert 16 // 4 == nf4["fp16_over_code_bits"]


def test_codebook_psumbook_equals_dequant_and_reduces_to_w2(golden_dir):
    c = synth.codebook_case(17, 3, 12, 512)
    y, A = ref.gemv_codebook(c["x"], c["codes"], c["codebook"], c["scales"])
    yp = ref.gemv_codebook_psumbook(c["x"], c["codes"], c["codebook"], c["scales"])
    assert np.all(np.abs(y - yp) <= 1e-12 * A)
    P = ref.psumbook(c["x"], c["codebook"])
    with open(os.path.join(golden_dir, "page_facts.json")) as f:
        facts = json.load(f)
    for e in facts["psumbook_entries_per_tile"]["cases"]:
        assert (e["t_w"] // e["v"]) * (2 ** e["b"]) * e["m"] == e["entries"]
    assert P.shape == (3, 512 // 4, 256)
    rc = facts["codebook_read_cost"]["cases"][0]
    assert rc["m"] * rc["rows"] * rc["K"] // rc["v"] * rc["batch"] == rc["reads"]
    # reduction to W2: centroid c holds the four 2-bit fields of c minus z0
    z0 = 1
    C = np.array([[((cc >> (2 * t)) & 3) - z0 for t in range(4)] for cc in range(256)], dtype=np.float16)
    yc, _ = ref.gemv_codebook(c["x"], c["codes"], C, c["scales"])
    q2 = np.zeros((12, 512), dtype=np.uint8)
    for t in range(4):
        q2[:, t::4] = (c["codes"] >> (2 * t)) & 3
    yu, Au = ref.gemv_uniform(c["x"], q2, c["scales"], np.full((12, 4), z0, dtype=np.uint8))
    assert np.all(np.abs(yc - yu) <= 1e-12 * Au)
    # one-hot x picks s * C[code][t]
    x = np.zeros((1, 512), dtype=np.float16); x[0, 4 * 37 + 2] = 1.0
    y1, _ = ref.gemv_codebook(x, c["codes"], c["codebook"], c["scales"])
    want = c["scales"][:, 1].astype(np.float64) * c["codebook"][c["codes"][:, 37], 2].astype(np.float64)
    assert np.array_equal(y1[0], want)


def test_outlier_special_cases():
    c = synth.outlier_case(18, 2, 16, 256, frac=0.03)
    none = np.zeros(0, dtype=np.int32)
    y0, A0 = ref.gemv_outlier(c["x"], c["codes"], c["scales"], c["zeros"], none, none,
                              np.zeros(0, dtype=np.float16))
    yu, Au = ref.gemv_uniform(c["x"], c["codes"], c["scales"], c["zeros"])
    assert np.array_equal(y0, yu) and np.array_equal(A0, Au)
    # zero scales leave a pure sparse product
    s0 = np.zeros_like(c["scales"])
    ys, _ = ref.gemv_outlier(c["x"], c["codes"], s0, c["zeros"], c["o_rows"], c["o_cols"], c["o_vals"])
    ye = exact.to_f64(exact.sparse_exact(c["x"], 16, c["o_rows"], c["o_cols"], c["o_vals"]))
    assert np.array_equal(ys, ye)
    # a single outlier under one-hot x adds v to s(q - z)
    x = np.zeros((1, 256), dtype=np.float16); x[0, 200] = 1.0
    y1, _ = ref.gemv_outlier(x, c["codes"], c["scales"], c["zeros"], [3], [200],
                             np.array([0.75], dtype=np.float16))
    w = float(c["scales"][3, 1]) * (int(c["codes"][3, 200]) - int(c["zeros"][3, 1]))
    assert y1[0, 3] == w + 0.75


def test_kernel_rounding_budget_fits_tolerance():
    """Emulate every rounding the reading permits (fp16 dequantized weight, fp32
    partial sums in an arbitrary order, fp16 output) and check the tolerance
    still holds with margin on a realistic shape: the reading is not too tight."""
    c = synth.uniform_case(19, 2, 256, 4096, 4)
    y_ref, A = ref.gemv_uniform(c["x"], c["codes"], c["scales"], c["zeros"])
    w16 = ref.dequant_uniform(c["codes"], c["scales"], c["zeros"]).astype(np.float16).astype(np.float32)
    prod = c["x"].astype(np.float32)[:, None, :] * w16[None, :, :]      # [M, N, K] fp32
    acc = np.zeros(prod.shape[:2], dtype=np.float32)
    for kk in range(0, 4096, 32):                                       # lane-split partials
        acc = acc + prod[:, :, kk:kk + 32].sum(axis=2, dtype=np.float32)
    y = acc.astype(np.float16)
    assert ref.worst_ratio(y, y_ref, A) < 0.6


# ----------------------------------------------------------------------------
# planted mistakes: a wrong oracle must fail a pin
# ----------------------------------------------------------------------------
def _mut_sign(codes, scales, zeros, g=128):
    return np.repeat(scales.astype(np.float64), g, 1) * (codes.astype(np.float64) + np.repeat(zeros.astype(np.float64), g, 1))


def _mut_group_off(codes, scales, zeros, g=128):
    s = np.roll(np.repeat(scales.astype(np.float64), g, 1), 1, axis=1)
    return s * (codes.astype(np.float64) - np.repeat(zeros.astype(np.float64), g, 1))


def _mut_dropped_zero(codes, scales, zeros, g=128):
    return np.repeat(scales.astype(np.float64), g, 1) * codes.astype(np.float64)


def _mut_transpose_groups(codes, scales, zeros, g=128):
    # zero point indexed by row of the group instead of the group
    z = np.repeat(zeros.astype(np.float64)[:, ::-1], g, 1)
    return np.repeat(scales.astype(np.float64), g, 1) * (codes.astype(np.float64) - z)


@pytest.mark.parametrize("mutant", [_mut_sign, _mut_group_off, _mut_dropped_zero, _mut_transpose_groups])
def test_planted_mistakes_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(ref, "dequant_uniform", mutant)
    failures = 0
    for pin in (lambda: test_uniform_matches_exact(4, 3, 5, 256),
                lambda: test_one_hot_x_gives_single_dequantized_weight(4),
                lambda: test_codes_equal_zero_points_give_zero(4)):
        try:
            pin()
        except AssertionError:
            failures += 1
    assert failures >= 1


# ----------------------------------------------------------------------------
# unfused baselines: the plain fp16 product and the additive sparse step
# ----------------------------------------------------------------------------
def test_dense_gemv_worked_example():
    """By hand: x = (1, 2, -1, 0.5, 0, ...), W rows (2, -1, 3, 4, 0, ...) and
    (0.25, 0.5, 0, -2, 0, ...): y = (2 - 2 - 3 + 2, 0.25 + 1 + 0 - 1) = (-1, 0.25),
    A = (2 + 2 + 3 + 2, 0.25 + 1 + 0 + 1) = (9, 2.25)."""
    K = 128
    x = np.zeros((1, K), np.float16)
    x[0, :4] = [1, 2, -1, 0.5]
    w = np.zeros((2, K), np.float16)
    w[0, :4] = [2, -1, 3, 4]
    w[1, :4] = [0.25, 0.5, 0, -2]
    y, A = ref.gemv_dense(x, w)
    assert y.tolist() == [[-1.0, 0.25]] and A.tolist() == [[9.0, 2.25]]


def test_dense_gemv_selects_columns():
    """A 0/1 weight with its one 1 of row n at column (5n + 3) mod K copies that
    column of x (a transposed, reversed or shifted operand fails)."""
    M, N, K = 3, 40, 128
    x = synth.activations(21, M, K)
    w = np.zeros((N, K), dtype=np.float16)
    cols = (5 * np.arange(N) + 3) % K
    w[np.arange(N), cols] = 1.0
    y, A = ref.gemv_dense(x, w)
    assert np.array_equal(y, x.astype(np.float64)[:, cols])
    assert np.array_equal(A, np.abs(y))


def test_dense_gemv_matches_exact_and_reduces_to_uniform():
    """Exact brute force on a tiny random case; and the eager chain's
    definition: the plain product over the dequantized weight is the uniform
    GEMV (pinned above), on all rows and on a row subset."""
    c = synth.dense_case(22, 2, 5, 128)
    y, A = ref.gemv_dense(c["x"], c["w"])
    ye = exact.to_f64(exact.gemv_dense_exact(c["x"], c["w"]))
    assert np.allclose(y, ye, rtol=0, atol=1e-12 * A.max())
    u = synth.uniform_case(23, 2, 24, 256, 4)
    w = ref.dequant_uniform(u["codes"], u["scales"], u["zeros"])
    yd, Ad = ref.gemv_dense(u["x"], w)
    yu, Au = ref.gemv_uniform(u["x"], u["codes"], u["scales"], u["zeros"])
    assert np.allclose(yd, yu, rtol=0, atol=1e-12 * Au.max()) and np.allclose(Ad, Au, rtol=1e-12)
    rows = [0, 7, 23]
    yr, Ar = ref.gemv_dense(u["x"], w, rows=rows)
    assert np.array_equal(yr, yd[:, rows]) and np.array_equal(Ar, Ad[:, rows])


def test_add_sparse_worked_example_and_special_cases():
    """By hand: x[1] = 2, x[200] = -1; prior y = (1, 1, 1, -0.5); outliers
    (row 2, col 1, 0.5), (2, 200, 0.25), (0, 200, 1.5):
    y = (1 - 1.5, 1, 1 + 1 - 0.25, -0.5), A = (1 + 1.5, 1, 1 + 1 + 0.25, 0.5)."""
    K = 256
    x = np.zeros((1, K), np.float16)
    x[0, 1], x[0, 200] = 2.0, -1.0
    yp = np.array([[1.0, 1.0, 1.0, -0.5]], np.float16)
    y, A = ref.add_sparse(yp, x, [2, 2, 0], [1, 200, 200], np.array([0.5, 0.25, 1.5], np.float16))
    assert y.tolist() == [[-0.5, 1.0, 1.75, -0.5]] and A.tolist() == [[2.5, 1.0, 2.25, 0.5]]
    none = np.zeros(0, np.int32)
    y0, _ = ref.add_sparse(yp, x, none, none, np.zeros(0, np.float16))
    assert np.array_equal(y0, yp.astype(np.float64))
    c = synth.outlier_case(24, 2, 32, 256, frac=0.03)
    ys, _ = ref.add_sparse(np.zeros((2, 32), np.float16), c["x"], c["o_rows"], c["o_cols"], c["o_vals"])
    assert np.array_equal(ys, exact.to_f64(exact.sparse_exact(c["x"], 32, c["o_rows"], c["o_cols"], c["o_vals"])))


def _dense_mut_reversed_k(x, w, rows=None):
    w = np.asarray(w)
    return ref._gemv_rows(ref._f64(x), lambda r: ref._f64(w[r])[:, ::-1], w.shape[0], rows)


def _dense_mut_signed_A(x, w, rows=None):
    x64, w64 = ref._f64(x), ref._f64(w)
    y = x64 @ w64.T
    return y, np.abs(y)


def _dense_mut_row_shift(x, w, rows=None):
    w = np.asarray(w)
    return ref._gemv_rows(ref._f64(x), lambda r: ref._f64(w[(r + 1) % w.shape[0]]), w.shape[0], rows)


@pytest.mark.parametrize("mutant", [_dense_mut_reversed_k, _dense_mut_signed_A, _dense_mut_row_shift])
def test_planted_dense_mistakes_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(ref, "gemv_dense", mutant)
    failures = 0
    for pin in (test_dense_gemv_worked_example, test_dense_gemv_selects_columns):
        try:
            pin()
        except AssertionError:
            failures += 1
    assert failures >= 1


# ----------------------------------------------------------------------------
# additive codebooks (m codebooks, vector length v, group g)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("m,v,g", [(1, 4, 32), (2, 8, 64), (3, 16, 32)])
def test_codebook_additive_matches_exact(m, v, g):
    c = synth.codebook_additive_case(25 + m, 2, 3, 128, m, v, g)
    y, A = ref.gemv_codebook_additive(c["x"], c["codes"], c["codebooks"], c["scales"], g)
    ye = exact.to_f64(exact.gemv_codebook_additive_exact(c["x"], c["codes"], c["codebooks"], c["scales"], g))
    assert np.allclose(y, ye, rtol=0, atol=1e-12 * A.max())


def test_codebook_additive_reduces_to_single_codebook():
    """m = 1 is the single-codebook format (pinned above), and a codebook of
    zeros adds nothing."""
    c = synth.codebook_additive_case(26, 2, 20, 512, 1, 4, 128)
    y1, A1 = ref.gemv_codebook_additive(c["x"], c["codes"], c["codebooks"], c["scales"], 128)
    ys, As = ref.gemv_codebook(c["x"], c["codes"][0], c["codebooks"][0], c["scales"], 128)
    assert np.array_equal(y1, ys) and np.array_equal(A1, As)
    c2 = synth.codebook_additive_case(27, 1, 20, 512, 2, 8, 64)
    cbs = c2["codebooks"].copy()
    cbs[1] = 0
    y2, _ = ref.gemv_codebook_additive(c2["x"], c2["codes"], cbs, c2["scales"], 64)
    ys2, _ = ref.gemv_codebook(c2["x"], c2["codes"][0], c2["codebooks"][0], c2["scales"], 64)
    assert np.allclose(y2, ys2, rtol=0, atol=1e-13)


def test_codebook_additive_one_hot_worked_example():
    """One-hot x at k = 37 (segment 2, dim 5 for v = 16; group 1 for g = 32):
    y[n] = s[n, 1] * (C_0[code_0[n, 2], 5] + C_1[code_1[n, 2], 5] + C_2[code_2[n, 2], 5])."""
    c = synth.codebook_additive_case(28, 1, 5, 128, 3, 16, 32)
    x = np.zeros((1, 128), np.float16)
    x[0, 37] = 1.0
    y, _ = ref.gemv_codebook_additive(x, c["codes"], c["codebooks"], c["scales"], 32)
    for n in range(5):
        w = float(c["scales"][n, 1]) * sum(float(c["codebooks"][i, int(c["codes"][i, n, 2]), 5]) for i in range(3))
        assert y[0, n] == pytest.approx(w, rel=1e-15, abs=0)


def _cb_mut_wrong_group(codes, codebooks, scales, g):
    return _orig_additive(codes, codebooks, np.roll(scales, 1, axis=1), g)


def _cb_mut_first_codebook_only(codes, codebooks, scales, g):
    return _orig_additive(codes[:1], codebooks[:1], scales, g)


_orig_additive = ref.dequant_codebook_additive


@pytest.mark.parametrize("mutant", [_cb_mut_wrong_group, _cb_mut_first_codebook_only])
def test_planted_codebook_mistakes_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(ref, "dequant_codebook_additive", mutant)
    with pytest.raises(AssertionError):
        test_codebook_additive_one_hot_worked_example()


# ----------------------------------------------------------------------------
# W4A8 (int8 activations, padding strategy)
# ----------------------------------------------------------------------------
def test_int8_activation_quantization_worked_example():
    """By hand: x = (1, -2, 0.5, fp16(2/127)): s = 2 / 127 (fp32); x / s =
    (63.5 exactly in fp32, -127, 31.75, 0.99994) -> rint, half to even =
    (64, -127, 32, 1); a zero row gives s = 0, q = 0."""
    x = np.zeros((2, 128), np.float16)
    x[0, :4] = [1.0, -2.0, 0.5, np.float16(2.0 / 127.0)]
    q, s = ref.quantize_activations_int8(x)
    assert s[0] == np.float32(2.0) / np.float32(127.0) and s[1] == 0
    assert q[0, :4].tolist() == [64, -127, 32, 1] and not q[0, 4:].any() and not q[1].any()


def test_w4a8_reduces_to_uniform_on_integer_activations():
    """Activations that are integers with max |x| = 127 quantize to themselves
    (s = 1), so W4A8 is the uniform GEMV on them."""
    c = synth.uniform_case(29, 3, 40, 256, 4)
    x = (np.arange(3 * 256).reshape(3, 256) % 255 - 127).astype(np.float16)
    y8, A8 = ref.gemv_w4a8(x, c["codes"], c["scales"], c["zeros"])
    yu, Au = ref.gemv_uniform(x, c["codes"], c["scales"], c["zeros"])
    assert np.array_equal(y8, yu) and np.array_equal(A8, Au)


def test_w4a8_within_quantization_error_of_w4a16():
    """|y_w4a8 - y_w4a16| <= (s_x / 2) * sum_k |w| (each activation moves by
    at most half a step), and the bound is not vacuous."""
    c = synth.uniform_case(30, 4, 64, 512, 4)
    y8, _ = ref.gemv_w4a8(c["x"], c["codes"], c["scales"], c["zeros"])
    y16, _ = ref.gemv_uniform(c["x"], c["codes"], c["scales"], c["zeros"])
    _, sx = ref.quantize_activations_int8(c["x"])
    wabs = np.abs(ref.dequant_uniform(c["codes"], c["scales"], c["zeros"])).sum(axis=1)
    bound = sx.astype(np.float64)[:, None] / 2 * wabs[None, :]
    assert (np.abs(y8 - y16) <= bound + 1e-12).all()
    assert np.abs(y8 - y16).max() > 0


# ----------------------------------------------------------------------------
# W4A8 with asymmetric activations (zero points on both operands) and the
# Split strategy
# ----------------------------------------------------------------------------
def test_asym8_quantization_worked_example():
    """By hand.  Row 0: x = (-3, 5, 0, 1, 0, ...): lo = -3, hi = 5, s = 8/255
    (fp32); lo/s = -95.625 -> rint -96, zx = -128 + 96 = -32; x/s = (-95.625,
    159.375, 0, 31.875) -> (-96, 159, 0, 32) + zx = (-128, 127, -32, 0).
    Row 1, constant 2 (the range widened to [0, 2]): s = 2/255, zx = -128,
    2/s -> 255, q = 127.  Row 2, zeros: s = 0, zx = 0, q = 0."""
    x = np.zeros((3, 128), np.float16)
    x[0, :4] = [-3.0, 5.0, 0.0, 1.0]
    x[1, :] = 2.0
    q, s, zx = ref.quantize_activations_asym8(x)
    assert s[0] == np.float32(8.0) / np.float32(255.0) and s[1] == np.float32(2.0) / np.float32(255.0) and s[2] == 0
    assert zx.tolist() == [-32, -128, 0]
    assert q[0, :4].tolist() == [-128, 127, -32, 0] and (q[0, 4:] == -32).all()
    assert (q[1] == 127).all() and not q[2].any()


def test_asym8_expansion_equals_definition():
    """The zero-point expansion with raw codes and raw activation bytes (every
    term an exact integer) equals the dequantize-then-multiply definition."""
    for seed, (M, N, K) in enumerate([(1, 7, 128), (3, 33, 512), (16, 64, 1024)]):
        c = synth.uniform_case(700 + seed, M, N, K, 4)
        y, A = ref.gemv_w4a8_asym(c["x"], c["codes"], c["scales"], c["zeros"])
        ye = ref.gemv_w4a8_asym_expanded(c["x"], c["codes"], c["scales"], c["zeros"])
        assert np.abs(y - ye).max() <= 1e-12 * max(1.0, A.max())


def test_asym8_exact_brute_force():
    c = synth.uniform_case(710, 2, 3, 256, 4)
    xq, sx, zx = ref.quantize_activations_asym8(c["x"])
    y, _ = ref.gemv_w4a8_asym(c["x"], c["codes"], c["scales"], c["zeros"])
    for m in range(2):
        for n in range(3):
            tot = Fraction(0)
            for k in range(256):
                w = Fraction(float(c["scales"][n, k // 128])) * (int(c["codes"][n, k]) - int(c["zeros"][n, k // 128]))
                tot += w * (int(xq[m, k]) - int(zx[m]))
            assert abs(float(tot * Fraction(float(sx[m]))) - y[m, n]) <= 1e-12 * max(1.0, abs(y[m, n]))


def test_asym8_reduces_to_uniform_on_full_range_integers():
    """Integer activations that span exactly [-128, 127] quantize to
    themselves (s = 1, zx = 0), so the result is the uniform GEMV on them."""
    c = synth.uniform_case(720, 3, 40, 256, 4)
    x = (np.arange(3 * 256).reshape(3, 256) % 256 - 128).astype(np.float16)
    q, s, zx = ref.quantize_activations_asym8(x)
    assert (s == 1).all() and (zx == 0).all() and np.array_equal(q.astype(np.float16), x)
    ya, Aa = ref.gemv_w4a8_asym(x, c["codes"], c["scales"], c["zeros"])
    yu, Au = ref.gemv_uniform(x, c["codes"], c["scales"], c["zeros"])
    assert np.array_equal(ya, yu) and np.array_equal(Aa, Au)


def test_asym8_within_quantization_error_of_w4a16():
    """Each activation moves by at most one step s_x (half a step by
    rounding, plus the clamp at the top of the range), and the bound is not
    vacuous; an asymmetric row (all positive) uses the range better than the
    symmetric scheme."""
    c = synth.uniform_case(730, 4, 64, 512, 4)
    x = c["x"].astype(np.float64)
    x[3] = np.abs(x[3]) + 0.5
    x = x.astype(np.float16)
    ya, _ = ref.gemv_w4a8_asym(x, c["codes"], c["scales"], c["zeros"])
    y16, _ = ref.gemv_uniform(x, c["codes"], c["scales"], c["zeros"])
    _, sx, _ = ref.quantize_activations_asym8(x)
    wabs = np.abs(ref.dequant_uniform(c["codes"], c["scales"], c["zeros"])).sum(axis=1)
    assert (np.abs(ya - y16) <= sx.astype(np.float64)[:, None] * wabs[None, :] + 1e-12).all()
    assert np.abs(ya - y16).max() > 0
    ys, _ = ref.gemv_w4a8(x, c["codes"], c["scales"], c["zeros"])
    assert np.abs(ya - y16)[3].max() < np.abs(ys - y16)[3].max()


def test_split_decomposition_is_exact():
    v = np.arange(-128, 128)
    h, l = ref.split_activations_int8(v)
    assert np.array_equal(16 * h + l, v)
    assert h.min() == -8 and h.max() == 7 and l.min() == 0 and l.max() == 15


def test_split_equals_padding():
    for seed, (M, N, K) in enumerate([(1, 9, 128), (5, 40, 640), (16, 32, 2048)]):
        c = synth.uniform_case(740 + seed, M, N, K, 4)
        ys, As = ref.gemv_w4a8_split(c["x"], c["codes"], c["scales"], c["zeros"])
        yp, Ap = ref.gemv_w4a8(c["x"], c["codes"], c["scales"], c["zeros"])
        assert np.abs(ys - yp).max() <= 1e-12 * max(1.0, Ap.max()) and np.array_equal(As, Ap)


def _mut_expansion_sign(x, codes, scales, zeros, g=128):
    xq, sx, zx = ref.quantize_activations_asym8(x)
    return ref.gemv_uniform(xq.astype(np.float64) + zx[:, None], codes, scales, zeros, g)[0] * sx.astype(np.float64)[:, None]


def test_planted_asym_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(ref, "gemv_w4a8_asym_expanded", _mut_expansion_sign)
    with pytest.raises(AssertionError):
        test_asym8_expansion_equals_definition()
