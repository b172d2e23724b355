"""CPU decoder of the library's packed activation rows (hi/lo FP6 E2M3 + E8M0).

Format (documented in include/moe_mxfp4.h): per row of K values
  [hi codes K/32 x 24 B][lo codes K/32 x 24 B][hi scales 2 x KTp][lo scales 2 x KTp],
KTp = roundup(K/64, 4); block b's codes are 6-bit fields, element i at bits
6i..6i+5 (little-endian); block b's scale byte sits at [b % 2][b // 2].
E2M3: sign bit 5, exponent bits 4-3 (bias 1), mantissa bits 2-0.
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
    ktp = (K // 64 + 3) // 4 * 4
    return K // 32 * 48 + 4 * ktp


def decode(buf, K: int, rows: int):
    """buf: uint8 array (at least rows*row_bytes(K)) -> (hi, lo) float64 [rows][K]."""
    nb = K // 32
    ktp = (K // 64 + 3) // 4 * 4
    rb = row_bytes(K)
    a = np.asarray(buf, dtype=np.uint8)[: rows * rb].reshape(rows, rb)
    out = []
    for term in range(2):
        codes = a[:, term * nb * 24:(term + 1) * nb * 24].reshape(rows, nb, 24)
        bits = np.unpackbits(codes, axis=2, bitorder="little").reshape(rows, nb, 32, 6)
        c = (bits * (1 << np.arange(6))).sum(axis=3)
        so = nb * 48 + term * 2 * ktp
        sc = a[:, so:so + 2 * ktp].reshape(rows, 2, ktp)
        b = np.arange(nb)
        sbyte = sc[:, b % 2, b // 2].astype(np.int64)                  # [rows][nb]
        val = _E2M3[c] * np.ldexp(1.0, sbyte - 127)[..., None]
        out.append(val.reshape(rows, K))
    return out[0], out[1]


def decode_sum(buf, K: int, rows: int) -> np.ndarray:
    hi, lo = decode(buf, K, rows)
    return hi + lo
