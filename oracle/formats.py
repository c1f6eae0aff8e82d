"""Storage formats, written as plain bit loops (oracle side; test infrastructure).

Plain packing (the weight format of the uniform and LUT variants)
----------------------------------------------------------------
The workloads store b-bit codes "packed 32/b per uint32 along K".  Reading
taken: code ``c`` of a row goes to word ``c // (32/b)`` of that row, in bits
``[b*(c % (32/b)), +b)`` -- the lowest k in the lowest bits.  A row occupies
``ceil(cols*b/32)`` words; unused high bits of a row's last word are zero.
Zero points use the same packing along the group axis.

Device packing (what the GEMV kernels read)
-------------------------------------------
Field order inside a word: a word covers P = 32/b consecutive k; field f holds
k offset 2f for f < P/2 and 2(f - P/2) + 1 for f >= P/2, so fields f and
f + P/2 hold two consecutive k and the two 16-bit halves of a word give (k, k+1)
pairs directly.  For b = 4 the fields hold k offsets 0,2,4,6,1,3,5,7.
``pack_device`` applies only this field order to the plain word sequence.

Tile order (``pack_tiles``, the weight format of the compute entry points):
the matrix is cut into tiles of 16 rows x 128 k (one quant group), padded with
code 0 to a multiple of 16 rows.  Tile (rt, g) occupies 16*128*b/32 words from
word (rt * G + g) * 64 * b (G = K / 128).  Inside a tile, "lane" l in [0, 64)
owns row 16*rt + (l % 16) and the 32 codes k in [128 g + 32 (l // 16), +32),
as b words in device field order (word i covers k offset (32/b)*i of that
run); lane l's word i sits at tile word (i // 4) * 256 + l * min(b, 4) + i % 4.
A wave-wide load of one word group per lane is then one contiguous block.

Tile-COO (outlier variant; FlashQuant abstract: "Tile-COO outlier encoding")
---------------------------------------------------------------------------
The page names the encoding but gives no fields.  Reading taken: tiles of
16 rows x 128 k -- the tile of the dense layout, one quant group of 16 rows --
numbered row-tile-major then k-tile (``t = (r // 16) * ceil(K/128) + c // 128``);
one uint32 per outlier with bits 0-7 = local column, bits 8-15 = local row,
bits 16-31 = the fp16 bits of the value; records sorted by (tile, local row,
local col); ``tile_ptr`` is the exclusive prefix sum of per-tile counts
(length tiles + 1).

Codebook code tiles (codebook variant)
--------------------------------------
uint8 codes ``[N, K/4]`` (one code per 4 consecutive k) are regrouped into
tiles of 64 rows x 16 code columns (1 KB).  Inside a tile, byte ``16*l + i``
(l = 0..63, i = 0..15) holds the code of row ``64*rt + l``, code column
``16*ct + i``.  Tiles are ordered row-tile-major, then column tile.  Rows and
columns past the matrix hold code 0.  (The device layout is the
implementation's choice; no page defines one.)
"""
from __future__ import annotations

import numpy as np


def words_per_row(cols: int, bits: int) -> int:
    return (cols * bits + 31) // 32


def pack_plain(codes: np.ndarray, bits: int) -> np.ndarray:
    """[R, C] uint8 codes -> [R, ceil(C*b/32)] uint32, one bit at a time."""
    codes = np.asarray(codes)
    if codes.ndim != 2:
        raise ValueError("codes must be 2-D")
    if bits not in (2, 4, 8):
        raise ValueError("bits must be 2, 4 or 8")
    if codes.size and int(codes.max()) >= (1 << bits):
        raise ValueError("code out of range")
    R, C = codes.shape
    per = 32 // bits
    out = np.zeros((R, words_per_row(C, bits)), dtype=np.uint64)
    c64 = codes.astype(np.uint64)
    for c in range(C):
        word = c // per
        base = bits * (c % per)
        for t in range(bits):
            bit = (c64[:, c] >> np.uint64(t)) & np.uint64(1)
            out[:, word] |= bit << np.uint64(base + t)
    return out.astype(np.uint32)


def unpack_plain(packed: np.ndarray, bits: int, cols: int) -> np.ndarray:
    """Inverse of pack_plain, one bit at a time."""
    packed = np.asarray(packed, dtype=np.uint32).astype(np.uint64)
    R = packed.shape[0]
    per = 32 // bits
    out = np.zeros((R, cols), dtype=np.uint64)
    for c in range(cols):
        word = c // per
        base = bits * (c % per)
        for t in range(bits):
            bit = (packed[:, word] >> np.uint64(base + t)) & np.uint64(1)
            out[:, c] |= bit << np.uint64(t)
    return out.astype(np.uint8)


def device_field_k(bits: int, f: int) -> int:
    """k offset (inside its word) of field f of a device-packed word."""
    half = (32 // bits) // 2
    return 2 * f if f < half else 2 * (f - half) + 1


def pack_device(codes: np.ndarray, bits: int) -> np.ndarray:
    """[R, C] uint8 codes -> device-packed [R, ceil(C*b/32)] uint32, bit by bit."""
    codes = np.asarray(codes)
    if codes.ndim != 2 or bits not in (2, 4, 8):
        raise ValueError("bad codes or bits")
    if codes.size and int(codes.max()) >= (1 << bits):
        raise ValueError("code out of range")
    R, C = codes.shape
    per = 32 // bits
    out = np.zeros((R, words_per_row(C, bits)), dtype=np.uint64)
    c64 = codes.astype(np.uint64)
    for j in range(out.shape[1]):
        for f in range(per):
            c = j * per + device_field_k(bits, f)
            if c >= C:
                continue
            for t in range(bits):
                bit = (c64[:, c] >> np.uint64(t)) & np.uint64(1)
                out[:, j] |= bit << np.uint64(bits * f + t)
    return out.astype(np.uint32)


def unpack_device(packed: np.ndarray, bits: int, cols: int) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint32).astype(np.uint64)
    R = packed.shape[0]
    per = 32 // bits
    out = np.zeros((R, cols), dtype=np.uint64)
    for j in range(packed.shape[1]):
        for f in range(per):
            c = j * per + device_field_k(bits, f)
            if c >= cols:
                continue
            for t in range(bits):
                bit = (packed[:, j] >> np.uint64(bits * f + t)) & np.uint64(1)
                out[:, c] |= bit << np.uint64(t)
    return out.astype(np.uint8)


def tiles_words(bits: int, rows: int, cols: int) -> int:
    return ((rows + 15) // 16) * 16 * cols * bits // 32


def pack_tiles(codes: np.ndarray, bits: int) -> np.ndarray:
    """[R, C] uint8 codes (C % 128 == 0) -> flat uint32 tile-order words."""
    codes = np.asarray(codes)
    R, C = codes.shape
    if C % 128:
        raise ValueError("cols must be a multiple of 128")
    per = 32 // bits
    G = C // 128
    RT = (R + 15) // 16
    pad = np.zeros((RT * 16, C), dtype=np.uint8)
    pad[:R] = codes
    rowwords = pack_device(pad, bits)             # [RT*16, C/per], field order applied
    out = np.zeros(tiles_words(bits, R, C), dtype=np.uint32)
    wpl = bits                                     # words per lane per tile
    for rt in range(RT):
        for g in range(G):
            base = (rt * G + g) * 64 * bits
            for l in range(64):
                r = 16 * rt + (l % 16)
                k0 = 128 * g + 32 * (l // 16)
                for i in range(wpl):
                    out[base + (i // 4) * 256 + l * min(bits, 4) + i % 4] = rowwords[r, (k0 + per * i) // per]
    return out


def unpack_tiles(words: np.ndarray, bits: int, rows: int, cols: int) -> np.ndarray:
    per = 32 // bits
    G = cols // 128
    RT = (rows + 15) // 16
    rowwords = np.zeros((RT * 16, cols // per), dtype=np.uint32)
    for rt in range(RT):
        for g in range(G):
            base = (rt * G + g) * 64 * bits
            for l in range(64):
                r = 16 * rt + (l % 16)
                k0 = 128 * g + 32 * (l // 16)
                for i in range(bits):
                    rowwords[r, (k0 + per * i) // per] = words[base + (i // 4) * 256 + l * min(bits, 4) + i % 4]
    return unpack_device(rowwords, bits, cols)[:rows]


# ----------------------------------------------------------------------------
# Tile-COO
# ----------------------------------------------------------------------------
TILE_R, TILE_C = 16, 128


def tilecoo_encode(N, K, rows, cols, vals_f16):
    """COO triplets -> (tile_ptr uint32[T+1], tile_rec uint32[nnz])."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    vals = np.asarray(vals_f16, dtype=np.float16)
    if not (rows.shape == cols.shape == vals.shape):
        raise ValueError("length mismatch")
    if rows.size and (rows.min() < 0 or rows.max() >= N or cols.min() < 0 or cols.max() >= K):
        raise ValueError("coordinate out of range")
    if len(set(zip(rows.tolist(), cols.tolist()))) != rows.size:
        raise ValueError("duplicate coordinate")
    if rows.size and not np.all(np.isfinite(vals.astype(np.float64))):
        raise ValueError("non-finite outlier value")
    KT = (K + TILE_C - 1) // TILE_C
    NT = (N + TILE_R - 1) // TILE_R
    entries = []
    for r, c, v in zip(rows.tolist(), cols.tolist(), vals.view(np.uint16).tolist()):
        t = (r // TILE_R) * KT + c // TILE_C
        lr, lc = r % TILE_R, c % TILE_C
        entries.append((t, lr, lc, (v << 16) | (lr << 8) | lc))
    entries.sort()
    counts = [0] * (NT * KT)
    for t, _, _, _ in entries:
        counts[t] += 1
    ptr = [0]
    for n in counts:
        ptr.append(ptr[-1] + n)
    return (np.array(ptr, dtype=np.uint32),
            np.array([e[3] for e in entries], dtype=np.uint32))


def tilecoo_decode(N, K, tile_ptr, tile_rec):
    """(tile_ptr, tile_rec) -> (rows int64, cols int64, vals fp16) in record order."""
    KT = (K + TILE_C - 1) // TILE_C
    rows, cols, vals = [], [], []
    for t in range(len(tile_ptr) - 1):
        tr, tk = divmod(t, KT)
        for i in range(int(tile_ptr[t]), int(tile_ptr[t + 1])):
            rec = int(tile_rec[i])
            rows.append(tr * TILE_R + ((rec >> 8) & 0xFF))
            cols.append(tk * TILE_C + (rec & 0xFF))
            vals.append(rec >> 16)
    return (np.array(rows, dtype=np.int64), np.array(cols, dtype=np.int64),
            np.array(vals, dtype=np.uint16).view(np.float16))


# ----------------------------------------------------------------------------
# codebook code tiles
# ----------------------------------------------------------------------------
CB_ROWS = 64  # rows per tile
CB_COLS = 16  # code columns per tile


def cb_tiled_bytes(N, KC):
    nr = (N + CB_ROWS - 1) // CB_ROWS
    nc = (KC + CB_COLS - 1) // CB_COLS
    return nr * nc * CB_ROWS * CB_COLS


def pack_codebook_tiles(codes: np.ndarray) -> np.ndarray:
    """[N, KC] uint8 -> flat uint8 tiles; byte 16*l + i of tile (rt, ct) holds
    code[64*rt + l, 16*ct + i]; out-of-range rows/columns hold 0."""
    N, KC = codes.shape
    NR = (N + CB_ROWS - 1) // CB_ROWS
    NC = (KC + CB_COLS - 1) // CB_COLS
    out = np.zeros(cb_tiled_bytes(N, KC), dtype=np.uint8)
    for rt in range(NR):
        for ct in range(NC):
            base = (rt * NC + ct) * CB_ROWS * CB_COLS
            for l in range(CB_ROWS):
                for i in range(CB_COLS):
                    r = rt * CB_ROWS + l
                    c = ct * CB_COLS + i
                    if r < N and c < KC:
                        out[base + CB_COLS * l + i] = codes[r, c]
    return out


def unpack_codebook_tiles(tiles: np.ndarray, N, KC) -> np.ndarray:
    NR = (N + CB_ROWS - 1) // CB_ROWS
    NC = (KC + CB_COLS - 1) // CB_COLS
    out = np.zeros((N, KC), dtype=np.uint8)
    for rt in range(NR):
        for ct in range(NC):
            base = (rt * NC + ct) * CB_ROWS * CB_COLS
            for l in range(CB_ROWS):
                for i in range(CB_COLS):
                    r = rt * CB_ROWS + l
                    c = ct * CB_COLS + i
                    if r < N and c < KC:
                        out[r, c] = tiles[base + CB_COLS * l + i]
    return out
