"""Pins for the acceptance predicate and for the kernels' fp32 arithmetic
(CPU only; test infrastructure).

1. ``within_tolerance`` / ``worst_ratio`` implement |y - y_ref| <= 2e-3 * A
   + 1e-6 exactly: the bound itself passes, the next float64 value fails, the
   relative and absolute terms are not swapped, NaN fails, and fp16 inputs are
   widened exactly.

2. The W4 VALU engine's arithmetic, emulated in float32 on the CPU: unpacked
   (q - z) pairs (exact small integers in fp16), a v_dot2_f32_f16 chain per
   lane over its 32 k of a group, the group scale applied with one fma per
   group, four k-quarters and the waves added in a fixed order, then fp16.
   The emulation passes the tolerance on random, near-degenerate and q == z
   inputs (where it is exactly 0).  The group identity
   sum s(q - z)x = s(sum q x - z sum x) (QFactory review, observation 2)
   evaluated the same way on the magic-number values 1024 + q fails the q == z
   case: its fp32 residue scales with 1024 * sum |x|, not with A.  That is why
   the kernels subtract the zero point exactly in fp16 before the dot product.
"""
import numpy as np
import pytest

import synth
from oracle import reference as ref

REL, ABS = 2e-3, 1e-6


# ----------------------------------------------------------------------------
# 1. the acceptance predicate
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("A", [0.0, 1e-9, 0.37, 1.0, 123.5, 4.0e4])
def test_bound_passes_and_next_value_fails(A):
    b = REL * A + ABS                              # the bound, as the predicate forms it
    y_ref = np.zeros((1, 2))
    AA = np.full((1, 2), A)
    on = np.array([[b, -b]])
    assert ref.within_tolerance(on, y_ref, AA).all()
    past = np.array([[np.nextafter(b, np.inf), -np.nextafter(b, np.inf)]])
    assert not ref.within_tolerance(past, y_ref, AA).any()
    assert ref.worst_ratio(on, y_ref, AA) <= 1.0 < ref.worst_ratio(past, y_ref, AA)


def test_relative_and_absolute_terms_not_swapped():
    y_ref = np.zeros((1, 1))
    # small A, error 1e-3: fails (2e-3 * 0.01 + 1e-6 = 2.1e-5), would pass swapped
    assert not ref.within_tolerance(np.array([[1e-3]]), y_ref, np.array([[0.01]])).any()
    # large A, error 0.1: passes (0.2 + 1e-6), would fail swapped (1e-4 + 2e-3)
    assert ref.within_tolerance(np.array([[0.1]]), y_ref, np.array([[100.0]])).all()
    # A = 0: only the absolute floor remains
    assert ref.within_tolerance(np.array([[1e-6]]), y_ref, np.zeros((1, 1))).all()
    assert not ref.within_tolerance(np.array([[1.1e-6]]), y_ref, np.zeros((1, 1))).any()


def test_nan_and_inf_fail_and_fp16_is_widened_exactly():
    y_ref = np.ones((1, 3))
    A = np.full((1, 3), 10.0)
    assert not ref.within_tolerance(np.array([[np.nan, np.inf, -np.inf]]), y_ref, A).any()
    # fp16 1.0009765625 (1 + 2^-10) is 9.77e-4 from 1: inside 2e-3 * 10 + 1e-6
    y16 = np.array([[1.0 + 2.0 ** -10] * 3], dtype=np.float16)
    assert ref.within_tolerance(y16, y_ref, A).all()
    # ... and outside the bound at A = 0.4 (8.01e-4), which a lossy widening could hide
    assert not ref.within_tolerance(y16, y_ref, np.full((1, 3), 0.4)).any()


# ----------------------------------------------------------------------------
# 2. the W4 VALU engine's fp32 arithmetic, emulated
# ----------------------------------------------------------------------------
def _dot2_chain(p, x):
    """A v_dot2_f32_f16 chain over pairs: acc = fp32(acc + p0 x0 + p1 x1),
    the fp16 x fp16 products exact; p, x: [..., 2 * npairs] float32."""
    acc = np.zeros(p.shape[:-1], dtype=np.float32)
    for i in range(0, p.shape[-1], 2):
        s = p[..., i].astype(np.float64) * x[..., i] + p[..., i + 1].astype(np.float64) * x[..., i + 1]
        acc = (acc.astype(np.float64) + s).astype(np.float32)
    return acc


def emulate_w4_valu(x, codes, scales, zeros, identity=False, waves=16):
    """y[n] for one activation row as the W4 VALU engine computes it: lane
    (row n, quarter kq) takes a dot2 chain over its 32 k of each group, then
    acc = fma(s, part, acc) in fp32; wave w takes groups w, w + waves, ...;
    the quarters are added (q0 + q2) + (q1 + q3) and the waves in order, then
    the sum is rounded to fp16.  identity=True evaluates each group as
    sum (1024 + q) x - (1024 + z) sum x instead of sum (q - z) x."""
    xf = x.astype(np.float32)[0]
    N, K = codes.shape
    G = K // 128
    accw = np.zeros((waves, 4, N), dtype=np.float32)
    for g in range(G):
        w = g % waves
        s = scales[:, g].astype(np.float32)
        z = zeros[:, g].astype(np.float32)
        for kq in range(4):
            k0 = 128 * g + 32 * kq
            xs = np.broadcast_to(xf[k0:k0 + 32], (N, 32))
            qq = codes[:, k0:k0 + 32].astype(np.float32)
            if identity:
                part = _dot2_chain(1024.0 + qq, xs)
                sx = _dot2_chain(np.ones((1, 32), np.float32), xf[None, k0:k0 + 32])[0]
                part = (part.astype(np.float64) - ((1024.0 + z).astype(np.float64) * sx)).astype(np.float32)
            else:
                part = _dot2_chain(qq - z[:, None], xs)
            accw[w, kq] = (s.astype(np.float64) * part + accw[w, kq]).astype(np.float32)
    lanes = (accw[:, 0] + accw[:, 2]) + (accw[:, 1] + accw[:, 3])   # [waves, N] fp32
    tot = np.zeros(N, dtype=np.float32)
    for w in range(waves):
        tot = tot + lanes[w]
    return tot.astype(np.float16)[None, :]


def _case(seed, N=32, K=4096):
    return synth.uniform_case(seed, 1, N, K, 4)


def test_plain_form_emulation_within_tolerance_on_random_inputs():
    c = _case(71)
    y = emulate_w4_valu(c["x"], c["codes"], c["scales"], c["zeros"])
    y_ref, A = ref.gemv_uniform(c["x"], c["codes"], c["scales"], c["zeros"])
    assert ref.worst_ratio(y, y_ref, A) < 0.5


def test_plain_form_emulation_exact_zero_when_codes_equal_zero_points():
    c = _case(72)
    codes = synth.degenerate_codes(72, c["zeros"], 4)
    y = emulate_w4_valu(c["x"], codes, c["scales"], c["zeros"])
    assert np.all(y.astype(np.float64) == 0.0)


def test_plain_form_emulation_within_tolerance_near_degenerate():
    c = _case(73)
    codes = synth.degenerate_codes(73, c["zeros"], 4, near=True)
    y = emulate_w4_valu(c["x"], codes, c["scales"], c["zeros"])
    y_ref, A = ref.gemv_uniform(c["x"], codes, c["scales"], c["zeros"])
    assert ref.within_tolerance(y, y_ref, A).all()


def test_identity_form_emulation_breaks_the_degenerate_case():
    """The reason the kernels do not evaluate the identity in fp32: with q == z
    the exact result is 0 (A = 0, bound 1e-6), and the identity's residue is
    far above it on most rows."""
    c = _case(72)
    codes = synth.degenerate_codes(72, c["zeros"], 4)
    y = emulate_w4_valu(c["x"], codes, c["scales"], c["zeros"], identity=True)
    y_ref, A = ref.gemv_uniform(c["x"], codes, c["scales"], c["zeros"])
    assert np.all(A == 0.0) and np.all(y_ref == 0.0)
    fails = ~ref.within_tolerance(y, y_ref, A)
    assert fails.sum() >= len(fails[0]) // 2
