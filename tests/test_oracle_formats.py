"""Pins for the oracle's storage formats (CPU only)."""
import json
import os

import numpy as np
import pytest

import synth
from oracle import formats


def _golden(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def test_plain_packing_golden_words(golden_dir):
    for case in _golden(golden_dir, "plain_packing.json")["cases"]:
        codes = np.array([case["codes"]], dtype=np.uint8)
        packed = formats.pack_plain(codes, case["bits"])
        assert packed.shape == (1, 1)
        assert int(packed[0, 0]) == int(case["word"], 16), case


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_plain_packing_integer_form_and_roundtrip(bits):
    rng = np.random.default_rng(bits)
    R, C = 5, 200  # C not a multiple of 32/b for b = 4, 8? 200 % 8 == 0; add ragged below
    for cols in (C, 37):
        codes = rng.integers(0, 1 << bits, size=(R, cols), dtype=np.uint8)
        packed = formats.pack_plain(codes, bits)
        per = 32 // bits
        assert packed.shape == (R, (cols + per - 1) // per)
        # integer closed form: word j = sum_i code[per*j + i] << (b*i)
        for r in range(R):
            for j in range(packed.shape[1]):
                want = 0
                for i in range(per):
                    c = per * j + i
                    if c < cols:
                        want |= int(codes[r, c]) << (bits * i)
                assert int(packed[r, j]) == want
        assert np.array_equal(formats.unpack_plain(packed, bits, cols), codes)


def test_device_packing_golden_words(golden_dir):
    for case in _golden(golden_dir, "plain_packing.json")["device_cases"]:
        codes = np.array([case["codes"]], dtype=np.uint8)
        packed = formats.pack_device(codes, case["bits"])
        assert int(packed[0, 0]) == int(case["word"], 16), case


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_device_packing_is_a_field_permutation_of_plain(bits):
    rng = np.random.default_rng(10 + bits)
    for cols in (256, 40):
        codes = rng.integers(0, 1 << bits, size=(4, cols), dtype=np.uint8)
        dev = formats.pack_device(codes, bits)
        plain = formats.pack_plain(codes, bits)
        assert dev.shape == plain.shape
        assert np.array_equal(formats.unpack_device(dev, bits, cols), codes)
        per = 32 // bits
        # fields f and f + per/2 of every word hold consecutive k
        for j in range(dev.shape[1]):
            for f in range(per // 2):
                k_lo = j * per + 2 * f
                if k_lo + 1 < cols:
                    lo = (int(dev[0, j]) >> (bits * f)) & ((1 << bits) - 1)
                    hi = (int(dev[0, j]) >> (bits * (f + per // 2))) & ((1 << bits) - 1)
                    assert (lo, hi) == (codes[0, k_lo], codes[0, k_lo + 1])
        # same multiset of fields per word as the plain packing
        for j in range(dev.shape[1]):
            fd = sorted((int(dev[1, j]) >> (bits * f)) & ((1 << bits) - 1) for f in range(per))
            fp = sorted((int(plain[1, j]) >> (bits * f)) & ((1 << bits) - 1) for f in range(per))
            assert fd == fp


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_tile_order_positions_and_roundtrip(bits):
    """Hand-derived positions of the tile order, then a round trip on a ragged shape."""
    R, C = 20, 256                      # 2 row tiles (second padded), 2 groups
    codes = ((np.arange(R)[:, None] * 5 + np.arange(C)[None, :] * 3) % (1 << bits)).astype(np.uint8)
    words = formats.pack_tiles(codes, bits)
    assert words.size == 32 * C * bits // 32
    per = 32 // bits
    # tile (rt=1, g=1), lane l = 16*kq + n: row 16 + n, k from 128 + 32*kq
    for n, kq, i in [(0, 0, 0), (3, 2, bits - 1), (15, 3, bits // 2)]:
        l = 16 * kq + n
        w = int(words[(1 * 2 + 1) * 64 * bits + (i // 4) * 256 + l * min(bits, 4) + i % 4])
        r, k = 16 + n, 128 + 32 * kq + per * i
        for f in range(per):
            kk = k + formats.device_field_k(bits, f)
            want = codes[r, kk] if r < R else 0
            assert (w >> (bits * f)) & ((1 << bits) - 1) == want, (n, kq, i, f)
    assert np.array_equal(formats.unpack_tiles(words, bits, R, C), codes)


def test_plain_packing_rejects_bad_codes():
    with pytest.raises(ValueError):
        formats.pack_plain(np.array([[4]], dtype=np.uint8), 2)
    with pytest.raises(ValueError):
        formats.pack_plain(np.array([[0]], dtype=np.uint8), 3)


def test_tilecoo_hand_example():
    # N=200 (13 row tiles of 16, the last ragged), K=256 (2 k tiles): 26 tiles
    rows = [130, 0, 5, 5, 199]
    cols = [255, 3, 200, 1, 0]
    vals = np.array([1.5, -2.0, 0.25, 3.0, -0.125], dtype=np.float16)
    ptr, rec = formats.tilecoo_encode(200, 256, rows, cols, vals)
    # tiles (row tile, k tile) -> t = 2 rt + kt:
    #   t0 = (0,0): (0,3), (5,1)   t1 = (0,1): (5,200)
    #   t17 = (8,1): (130,255)     t24 = (12,0): (199,0)
    want_ptr = [0, 2] + [3] * 16 + [4] * 7 + [5] * 2
    assert len(want_ptr) == 27 and ptr.tolist() == want_ptr
    vb = vals.view(np.uint16)
    want = [
        (int(vb[1]) << 16) | (0 << 8) | 3,
        (int(vb[3]) << 16) | (5 << 8) | 1,
        (int(vb[2]) << 16) | (5 << 8) | (200 - 128),
        (int(vb[0]) << 16) | ((130 - 128) << 8) | (255 - 128),
        (int(vb[4]) << 16) | ((199 - 192) << 8) | 0,
    ]
    assert rec.tolist() == want
    r2, c2, v2 = formats.tilecoo_decode(200, 256, ptr, rec)
    got = sorted(zip(r2.tolist(), c2.tolist(), v2.astype(np.float64).tolist()))
    assert got == sorted(zip(rows, cols, vals.astype(np.float64).tolist()))


def test_tilecoo_roundtrip_and_errors():
    case = synth.outlier_case(7, 1, 384, 512, frac=0.01)
    ptr, rec = formats.tilecoo_encode(384, 512, case["o_rows"], case["o_cols"], case["o_vals"])
    assert len(ptr) == 24 * 4 + 1 and int(ptr[-1]) == len(case["o_rows"])
    assert np.all(np.diff(ptr.astype(np.int64)) >= 0)
    r, c, v = formats.tilecoo_decode(384, 512, ptr, rec)
    a = sorted(zip(r.tolist(), c.tolist(), v.view(np.uint16).tolist()))
    b = sorted(zip(case["o_rows"].tolist(), case["o_cols"].tolist(),
                   case["o_vals"].view(np.uint16).tolist()))
    assert a == b
    with pytest.raises(ValueError):
        formats.tilecoo_encode(4, 4, [0, 0], [1, 1], np.array([1, 2], dtype=np.float16))
    with pytest.raises(ValueError):
        formats.tilecoo_encode(4, 4, [4], [0], np.array([1], dtype=np.float16))
    with pytest.raises(ValueError):
        formats.tilecoo_encode(4, 4, [0], [0], np.array([np.inf], dtype=np.float16))


def test_codebook_tiles_positions_and_roundtrip():
    N, KC = 70, 40  # ragged in both directions
    codes = ((np.arange(N)[:, None] * 7 + np.arange(KC)[None, :] * 3) % 256).astype(np.uint8)
    tiles = formats.pack_codebook_tiles(codes)
    assert tiles.size == 2 * 3 * 1024
    # tile (rt=1, ct=2) byte 16*l + i  <->  code[64 + l, 32 + i]
    base = (1 * 3 + 2) * 1024
    assert tiles[base + 16 * 5 + 3] == codes[69, 35]
    assert tiles[base + 16 * 0 + 7] == codes[64, 39]
    assert tiles[base + 16 * 0 + 8] == 0           # column 40 is past KC
    assert tiles[base + 16 * 6 + 0] == 0           # row 70 is past N
    # tile (rt=0, ct=0) byte 16*l + i  <->  code[l, i]
    assert tiles[16 * 63 + 15] == codes[63, 15]
    assert np.array_equal(formats.unpack_codebook_tiles(tiles, N, KC), codes)


def test_codebook_storage_matches_page(golden_dir):
    facts = _golden(golden_dir, "page_facts.json")["codebook_bits_per_weight"]["cases"]
    for f in facts:
        N, K = 64, 512
        KC = K // f["v"]
        code_bits = N * KC * f["b"] * f["m"]
        scale_bits = N * (K // f["g"]) * 16
        assert (code_bits + scale_bits) / (N * K) == pytest.approx(f["qbar"], abs=1e-12)
    # the tiled device layout adds no bytes for tile-aligned shapes
    assert formats.cb_tiled_bytes(64, 128) == 64 * 128
