"""The library's host-side Tile-COO encoder against the oracle's (bit-exact),
and its error handling.  CPU only: the encoder runs on host pointers."""
import os

import numpy as np
import pytest

import synth
from oracle import formats

q = pytest.importorskip("gemm_unpack_bit_amd")
if not os.path.exists(q.LIB_PATH):
    pytest.skip("library not built", allow_module_level=True)


# (4800, 30720): 72,000 tiles, past 16 bits of tile index
@pytest.mark.parametrize("N,K,frac", [(128, 128, 0.01), (300, 384, 0.005), (4096, 4096, 0.005), (129, 1000, 0.02),
                                      (4800, 30720, 0.0005)])
def test_encoder_matches_oracle(N, K, frac):
    nnz = int(frac * N * K)
    pos = synth.unique_positions(N + K, synth.S_OPOS, N * K, nnz)
    rows, cols = pos // K, pos % K
    vals = synth.f16(synth.normal(N + K, synth.S_OVAL, nnz, 0.2))
    ptr, rec = q.tilecoo_encode(N, K, rows, cols, vals)
    ptr_o, rec_o = formats.tilecoo_encode(N, K, rows, cols, vals)
    assert np.array_equal(ptr, ptr_o)
    assert np.array_equal(rec, rec_o)
    r2, c2, v2 = formats.tilecoo_decode(N, K, ptr, rec)
    order = np.lexsort((cols, rows))
    back = np.lexsort((c2, r2))
    assert np.array_equal(r2[back], rows[order]) and np.array_equal(c2[back], cols[order])
    assert np.array_equal(v2[back].view(np.uint16), vals[order].view(np.uint16))


def test_encoder_empty_and_unsorted_input():
    ptr, rec = q.tilecoo_encode(256, 256, [], [], [])
    assert ptr.tolist() == [0] * (16 * 2 + 1) and rec.size == 0  # 16 row tiles x 2 k tiles
    rows, cols = [5, 1, 200, 1], [300, 7, 2, 3]
    vals = np.array([1.5, -2, 0.25, 3], dtype=np.float16)
    ptr, rec = q.tilecoo_encode(256, 384, rows, cols, vals)
    ptr_o, rec_o = formats.tilecoo_encode(256, 384, rows, cols, vals)
    assert np.array_equal(ptr, ptr_o) and np.array_equal(rec, rec_o)


def test_encoder_rejects_bad_input():
    with pytest.raises(q.QgemvError) as e:
        q.tilecoo_encode(64, 64, [1, 1], [2, 2], np.array([1, 2], dtype=np.float16))
    assert e.value.status == q.ERR_VALUE                                     # repeated position
    with pytest.raises(q.QgemvError) as e:
        q.tilecoo_encode(64, 64, [64], [0], np.array([1], dtype=np.float16))
    assert e.value.status == q.ERR_VALUE                                     # row out of range
    with pytest.raises(q.QgemvError) as e:
        q.tilecoo_encode(64, 64, [0], [0], np.array([np.inf], dtype=np.float16))
    assert e.value.status == q.ERR_VALUE                                     # non-finite value
    with pytest.raises(ValueError):
        q.tilecoo_encode(0, 64, [], [], [])
