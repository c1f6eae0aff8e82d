"""Seeded synthetic inputs for the quantized GEMV workloads.

This module is the only code shared by the oracle side (``oracle/``, tests)
and the GPU side (bindings, bench).  It draws random numbers and nothing else:
it holds none of the method's arithmetic (no packing, no dequantization, no
products).  Every array it returns is the *logical* input: one code per byte,
fp16 values as ``numpy.float16``.

Random source: splitmix64 (Steele, Lea, Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014), evaluated in counter mode so any element can
be produced independently of the others:

    out[i] = mix64(state0 + (i + 1) * GAMMA)

with ``state0 = mix64((seed << 8) | stream_id)``.  Uniforms in [0,1) take the
top 53 bits; b-bit codes take consecutive b-bit fields of each 64-bit output;
normals use the Box-Muller cosine branch on two uniforms; every real value is
drawn in float64 and rounded once to fp16 (round to nearest even), and that
rounded value *is* the input.

Workload recipes (distributions, shapes) follow the configurations of the
surveyed kernels: group-wise asymmetric W2/W4/W8 with g=128, a 16-entry
normal-quantile LUT with per-64 absmax, 0.5% fp16 outliers, and an m=1 v=4
b=8 codebook with per-128 scales.
"""
from __future__ import annotations

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

# sub-stream identifiers (fixed, so that every consumer draws the same bytes)
S_X, S_CODES, S_SCALES, S_ZEROS, S_OPOS, S_OVAL, S_CB, S_LUT, S_W, S_Y = range(1, 11)


def _mix64(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def _state0(seed: int, stream_id: int) -> np.uint64:
    s = ((int(seed) << 8) | int(stream_id)) & 0xFFFFFFFFFFFFFFFF
    return _mix64(np.array([s], dtype=np.uint64))[0]


def words(seed: int, stream_id: int, n: int, start: int = 0) -> np.ndarray:
    """n consecutive splitmix64 outputs (uint64) of one sub-stream, from index start."""
    st = _state0(seed, stream_id)
    idx = np.arange(start + 1, start + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix64(st + idx * GAMMA)


def uniform01(seed: int, stream_id: int, n: int, start: int = 0) -> np.ndarray:
    w = words(seed, stream_id, n, start)
    return (w >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def uniform(seed, stream_id, n, lo, hi, start=0) -> np.ndarray:
    return lo + (hi - lo) * uniform01(seed, stream_id, n, start)


def normal(seed, stream_id, n, std=1.0, start=0) -> np.ndarray:
    """Box-Muller (cosine branch): element i uses uniforms 2i and 2i+1."""
    u = uniform01(seed, stream_id, 2 * n, 2 * start)
    u1 = 1.0 - u[0::2]  # (0, 1]
    u2 = u[1::2]
    return std * np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)


def codes(seed, stream_id, n, bits) -> np.ndarray:
    """n uniform b-bit codes (uint8): code i = bits [b*(i % per), +b) of word i // per."""
    per = 64 // bits
    nw = (n + per - 1) // per
    w = words(seed, stream_id, nw)
    out = np.empty((nw, per), dtype=np.uint8)
    mask = np.uint64((1 << bits) - 1)
    for t in range(per):
        out[:, t] = ((w >> np.uint64(bits * t)) & mask).astype(np.uint8)
    return out.reshape(-1)[:n]


def f16(a) -> np.ndarray:
    """Round float64 values to fp16 (numpy rounds double->half to nearest even)."""
    return np.asarray(a, dtype=np.float64).astype(np.float16)


def seed_for(config: int, shape_index: int) -> int:
    return 0x5EED0000 + 256 * config + shape_index


# ----------------------------------------------------------------------------
# workload recipes
# ----------------------------------------------------------------------------

def activations(seed, M, K) -> np.ndarray:
    return f16(normal(seed, S_X, M * K)).reshape(M, K)


def uniform_case(seed, M, N, K, bits, g=128, s_lo=0.001, s_hi=0.02):
    """Group-wise asymmetric case: x ~ N(0,1); codes, zeros ~ U{0..2^b-1};
    scales ~ U(s_lo, s_hi); one scale and one zero per (row, g consecutive k)."""
    assert K % g == 0
    G = K // g
    return dict(
        x=activations(seed, M, K),
        codes=codes(seed, S_CODES, N * K, bits).reshape(N, K),
        scales=f16(uniform(seed, S_SCALES, N * G, s_lo, s_hi)).reshape(N, G),
        zeros=codes(seed, S_ZEROS, N * G, bits).reshape(N, G),
        bits=bits,
    )


def degenerate_codes(seed, zeros, bits, g=128, near=False):
    """Codes equal to their group's zero point (q == z at every k: the exact
    product is 0).  With near=True, one code per (row, group), at a uniform
    position inside the group, is one step away from z (up, or down at the
    top code), so each group holds exactly one nonzero weight."""
    zeros = np.asarray(zeros)
    N, G = zeros.shape
    out = np.repeat(zeros, g, axis=1).astype(np.uint8)
    if near:
        pos = (uniform01(seed, S_OPOS, N * G) * g).astype(np.int64).reshape(N, G)
        rows = np.arange(N)
        top = (1 << bits) - 1
        for j in range(G):
            k = g * j + pos[:, j]
            z = out[rows, k].astype(np.int64)
            out[rows, k] = np.where(z < top, z + 1, z - 1).astype(np.uint8)
    return out


def dense_case(seed, M, N, K, std=0.02):
    """fp16 weight [N, K] ~ N(0, std) (the magnitude of a dequantized weight)
    and activations x ~ N(0, 1): the input of a plain fp16 GEMV."""
    return dict(x=activations(seed, M, K), w=f16(normal(seed, S_W, N * K, std)).reshape(N, K))


def output_prior(seed, M, N, std=1.0) -> np.ndarray:
    """An fp16 [M, N] output already written by a dense kernel, ~ N(0, std)."""
    return f16(normal(seed, S_Y, M * N, std)).reshape(M, N)


def normal_quantile_levels(n=16) -> np.ndarray:
    """Levels Phi^-1((i+0.5)/n) / Phi^-1((n-0.5)/n), rounded to fp16 (runtime LUT input)."""
    from scipy.special import ndtri

    p = (np.arange(n, dtype=np.float64) + 0.5) / n
    return f16(ndtri(p) / ndtri((n - 0.5) / n))


def lut4_case(seed, M, N, K, block=64, a_lo=0.005, a_hi=0.05):
    assert K % block == 0
    return dict(
        x=activations(seed, M, K),
        codes=codes(seed, S_CODES, N * K, 4).reshape(N, K),
        absmax=f16(uniform(seed, S_SCALES, N * (K // block), a_lo, a_hi)).reshape(N, K // block),
        lut=normal_quantile_levels(16),
    )


def unique_positions(seed, stream_id, total, count) -> np.ndarray:
    """Floyd's algorithm: `count` distinct integers in [0, total), sorted (int64)."""
    if count > total:
        raise ValueError("count > total")
    u = uniform01(seed, stream_id, count)
    chosen = set()
    for i, j in enumerate(range(total - count, total)):
        t = int(u[i] * (j + 1))  # uniform in [0, j]
        chosen.add(j if t in chosen else t)
    return np.array(sorted(chosen), dtype=np.int64)


def outlier_case(seed, M, N, K, frac=0.005, std=0.2, bits=4):
    base = uniform_case(seed, M, N, K, bits)
    nnz = int(frac * N * K)
    pos = unique_positions(seed, S_OPOS, N * K, nnz)
    base.update(
        o_rows=(pos // K).astype(np.int32),
        o_cols=(pos % K).astype(np.int32),
        o_vals=f16(normal(seed, S_OVAL, nnz, std)),
    )
    return base


def codebook_case(seed, M, N, K, ncent=256, v=4, g=128, c_std=0.02, s_lo=0.5, s_hi=2.0):
    assert K % g == 0 and g % v == 0
    return dict(
        x=activations(seed, M, K),
        codes=codes(seed, S_CODES, N * (K // v), 8).reshape(N, K // v),
        codebook=f16(normal(seed, S_CB, ncent * v, c_std)).reshape(ncent, v),
        scales=f16(uniform(seed, S_SCALES, N * (K // g), s_lo, s_hi)).reshape(N, K // g),
    )


# Shapes named by the workloads (N = output features, K = reduction dim).
LLAMA3_8B_LAYERS = {
    "qkv": (6144, 4096),
    "o": (4096, 4096),
    "gate_up": (28672, 4096),
    "down": (4096, 14336),
}
LLAMA_70B_LAYERS = {
    "qkv": (10240, 8192),
    "o": (8192, 8192),
    "gate_up": (57344, 8192),
    "down": (8192, 28672),
}


def codebook_additive_case(seed, M, N, K, ncb, v, g, c_std=0.02, s_lo=0.5, s_hi=2.0):
    """ncb additive codebooks of 256 centroids of v dims: codes [ncb, N, K/v]
    uniform 8-bit, centroids [ncb, 256, v] ~ N(0, c_std), per-g scales."""
    assert K % g == 0 and g % v == 0
    return dict(
        x=activations(seed, M, K),
        codes=codes(seed, S_CODES, ncb * N * (K // v), 8).reshape(ncb, N, K // v),
        codebooks=f16(normal(seed, S_CB, ncb * 256 * v, c_std)).reshape(ncb, 256, v),
        scales=f16(uniform(seed, S_SCALES, N * (K // g), s_lo, s_hi)).reshape(N, K // g),
    )
