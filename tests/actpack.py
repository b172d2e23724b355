"""CPU decoder of the library's packed activation rows (hi/lo FP6 E2M3 + E8M0).

Format (documented in include/moe_mxfp4.h): per row of K values, K/64 chunks of
112 bytes, one per 64-wide k-tile kt: [0,24) hi codes of block 2kt, [24,48) hi
codes of block 2kt+1, [48,72) and [72,96) the lo codes, [96],[97] the hi scale
bytes and [98],[99] the lo scale bytes of blocks 2kt, 2kt+1.  Codes are 6-bit
fields, element i at bits 6i..6i+5 (little-endian).  E2M3: sign bit 5, exponent
bits 4-3 (bias 1), mantissa bits 2-0.
"""
import numpy as np


def e2m3_table() -> np.ndarray:
    t = np.zeros(64)
    for c in range(64):
        s = -1.0 if c & 32 else 1.0
        e, m = (c >> 3) & 3, c & 7
        t[c] = s * (m / 8.0 if e == 0 else 2.0 ** (e - 1) * (1 + m / 8.0))
    return t


_E2M3 = e2m3_table()


def row_bytes(K: int) -> int:
    return K // 64 * 112


def decode(buf, K: int, rows: int, chunk: int = 2048):
    """buf: uint8 array (at least rows*row_bytes(K)) -> (hi, lo) float64 [rows][K].
    Rows are decoded `chunk` at a time so the bit-level temporaries stay small."""
    kt = K // 64
    a = np.asarray(buf, dtype=np.uint8).reshape(-1)[: rows * row_bytes(K)].reshape(rows, kt, 112)
    hi, lo = np.empty((rows, K)), np.empty((rows, K))
    weights = (1 << np.arange(6)).astype(np.uint8)
    for r0 in range(0, rows, chunk):
        sub = a[r0:r0 + chunk]
        n = sub.shape[0]
        for term, dst in ((0, hi), (1, lo)):
            codes = sub[:, :, term * 48:(term + 1) * 48].reshape(n, kt, 2, 24)
            bits = np.unpackbits(codes, axis=3, bitorder="little").reshape(n, kt, 2, 32, 6)
            c = (bits * weights).sum(axis=4, dtype=np.int64)
            sbyte = sub[:, :, 96 + 2 * term:98 + 2 * term].astype(np.int64)    # [n][kt][2]
            dst[r0:r0 + n] = (_E2M3[c] * np.ldexp(1.0, sbyte - 127)[..., None]).reshape(n, K)
    return hi, lo


def decode_sum(buf, K: int, rows: int) -> np.ndarray:
    hi, lo = decode(buf, K, rows)
    return hi + lo


# ---- host encoder of the same format (CPU tests of the parity machinery) --------------------
# Written from the format description: per 32-value block, the shared exponent floor(log2 amax) - 2
# as an E8M0 byte clamped to [1, 253] (127 for an all-zero block); each value divided by the scale
# and rounded to the nearest E2M3 magnitude, ties to the even code, saturating at 7.5.  lo is the
# same encoding of what hi leaves over.
_E2M3_POS = _E2M3[:32]                     # codes 0..31: the non-negative magnitudes, ascending


def _scale_byte(amax: np.ndarray) -> np.ndarray:
    ex = np.frexp(np.where(amax > 0, amax, 1.0))[1] - 1 - 2       # floor(log2 amax) - 2
    return np.where(amax > 0, np.clip(ex + 127, 1, 253), 127).astype(np.int64)


def _e2m3_codes(q: np.ndarray) -> np.ndarray:
    """Nearest E2M3 code of each value (ties to the even code, magnitudes past 7.5 to 7.5)."""
    m = np.minimum(np.abs(q), 7.5)
    d = np.abs(m[..., None] - _E2M3_POS)
    best = d.min(axis=-1, keepdims=True)
    even = np.arange(32) % 2 == 0
    tie_even = (d == best) & even
    code = np.where(tie_even.any(axis=-1), np.argmax(tie_even, axis=-1), np.argmax(d == best, axis=-1))
    return code | np.where(q < 0, 32, 0)


def _split_block_terms(v: np.ndarray):
    """v [..., 32] -> (codes hi, codes lo, scale byte hi, scale byte lo)."""
    sh = _scale_byte(np.abs(v).max(-1))
    ch = _e2m3_codes(v / np.ldexp(1.0, sh - 127)[..., None])
    hi = _E2M3[ch] * np.ldexp(1.0, sh - 127)[..., None]
    r = v - hi
    sl = _scale_byte(np.abs(r).max(-1))
    cl = _e2m3_codes(r / np.ldexp(1.0, sl - 127)[..., None])
    return ch, cl, sh, sl


def encode(v: np.ndarray) -> np.ndarray:
    """Rows [R][K] of bf16 values (float64) -> packed bytes uint8 [R][row_bytes(K)]."""
    R, K = v.shape
    kt = K // 64
    ch, cl, sh, sl = _split_block_terms(np.asarray(v, np.float64).reshape(R, kt, 2, 32))
    out = np.zeros((R, kt, 112), np.uint8)
    for term, c in ((0, ch), (1, cl)):
        bits = ((c[..., None] >> np.arange(6)) & 1).astype(np.uint8).reshape(R, kt, 2, 192)
        out[:, :, term * 48:(term + 1) * 48] = np.packbits(bits, axis=-1, bitorder="little").reshape(R, kt, 48)
    out[:, :, 96:98] = sh
    out[:, :, 98:100] = sl
    return out.reshape(R, kt * 112)


# ---- MXFP4 activation rows (the activation-quantized entry points) -------------------------
# Per row, K/64 chunks of 48 bytes: [0,16) E2M1 codes of block 2kt (element i in nibble i, low
# nibble first), [16,32) codes of block 2kt+1, [32],[33] their E8M0 scale bytes.
def e2m1_table() -> np.ndarray:
    t = np.zeros(16)
    for c in range(16):
        s = -1.0 if c & 8 else 1.0
        e, m = (c >> 1) & 3, c & 1
        t[c] = s * (m / 2.0 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2.0))
    return t


_E2M1 = e2m1_table()


def row4_bytes(K: int) -> int:
    return K // 64 * 48


def decode4(buf, K: int, rows: int) -> np.ndarray:
    """buf: uint8 array (at least rows*row4_bytes(K)) -> float64 [rows][K]."""
    kt = K // 64
    a = np.asarray(buf, dtype=np.uint8)[: rows * row4_bytes(K)].reshape(rows, kt, 48)
    codes = a[:, :, :32].reshape(rows, kt, 2, 16)
    c = np.stack([codes & 0xF, codes >> 4], axis=-1).reshape(rows, kt, 2, 32)
    sbyte = a[:, :, 32:34].astype(np.int64)
    val = _E2M1[c] * np.ldexp(1.0, sbyte - 127)[..., None]
    return val.reshape(rows, K)
