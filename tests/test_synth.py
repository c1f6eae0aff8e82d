"""The seeded input generator: determinism, ranges and distribution recipe."""
import numpy as np

import synth


def test_splitmix64_reference_values():
    # splitmix64 published definition, counter mode from state0 = mix64(seed<<8 | stream)
    def mix(z):
        z &= (1 << 64) - 1
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & ((1 << 64) - 1)
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & ((1 << 64) - 1)
        return z ^ (z >> 31)

    st = mix((1234 << 8) | 3)
    want = [mix(st + (i + 1) * 0x9E3779B97F4A7C15) for i in range(5)]
    assert synth.words(1234, 3, 5).tolist() == want
    assert synth.words(1234, 3, 3, start=2).tolist() == want[2:5]


def test_deterministic_and_stream_separated():
    a = synth.uniform_case(1, 2, 16, 256, 4)
    b = synth.uniform_case(1, 2, 16, 256, 4)
    for k in ("x", "codes", "scales", "zeros"):
        assert np.array_equal(a[k], b[k])
    assert not np.array_equal(synth.words(1, 1, 8), synth.words(1, 2, 8))


def test_recipe_ranges_and_moments():
    c = synth.uniform_case(2, 1, 512, 4096, 4)
    assert c["x"].dtype == np.float16 and c["codes"].dtype == np.uint8
    assert c["codes"].max() == 15 and c["codes"].min() == 0
    s = c["scales"].astype(np.float64)
    assert s.min() >= 0.000999 and s.max() <= 0.0201
    x = c["x"].astype(np.float64)
    assert abs(x.mean()) < 0.05 and abs(x.std() - 1.0) < 0.05
    counts = np.bincount(c["codes"].reshape(-1), minlength=16)
    assert counts.min() > 0.9 * counts.mean()
    for bits in (2, 8):
        cc = synth.codes(3, 2, 100000, bits)
        assert cc.max() == (1 << bits) - 1


def test_outlier_positions_unique_and_counted():
    c = synth.outlier_case(4, 1, 256, 512)
    nnz = int(0.005 * 256 * 512)
    pos = c["o_rows"].astype(np.int64) * 512 + c["o_cols"]
    assert len(pos) == nnz and len(np.unique(pos)) == nnz
    v = c["o_vals"].astype(np.float64)
    assert abs(v.std() - 0.2) < 0.03


def test_codebook_and_lut_recipes():
    c = synth.codebook_case(5, 1, 64, 1024)
    assert c["codes"].shape == (64, 256) and c["codebook"].shape == (256, 4)
    s = c["scales"].astype(np.float64)
    assert s.min() >= 0.4995 and s.max() <= 2.001
    lc = synth.lut4_case(6, 1, 32, 256)
    assert lc["absmax"].shape == (32, 4) and lc["lut"].shape == (16,)
