"""FP8 weight decode (test infrastructure only).

Source: aiqre model page "Qwen3.8-27B-DFlash2", section "Memory": besides bf16 (3.6 GiB)
and int4 (0.9 GiB) the drafter's weights take 1.8 GiB in an 8-bit floating-point
format, one byte per parameter.  The page names no encoding and no scaling; the
reading taken is the OCP 8-bit floating-point format E4M3 with one scale per output
row of each matrix:

    code bits  s eeee mmm   (sign, 4 exponent bits with bias 7, 3 mantissa bits)
      e > 0:   (-1)^s (1 + m/8) 2^(e - 7)     (e = 15, m = 7 is NaN: no infinities)
      e = 0:   (-1)^s (m/8) 2^-6              (subnormal; code 0x80 is -0)
    largest finite magnitude 448 (e = 15, m = 6), smallest 2^-9.

A matrix [N rows][K cols] (y = x . W^T, K along the input) is stored as its N K codes
in row order (row n at byte n K), followed at byte N K by N little-endian float32
scales s_n:  w[n][k] = s_n * value(code[n][k]).  The scales add 4 bytes per row, so the
drafter stays at one byte per parameter.
"""
import numpy as np


def e4m3_value(code):
    """Value of one E4M3 code (int 0..255) as a Python float (NaN for the NaN codes)."""
    code = int(code)
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 15
    m = code & 7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def decode_codes(codes):
    """uint8 codes (any shape) -> float64 values of the same shape."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def split(data, rows, cols):
    """The codes [rows, cols] (uint8) and scales [rows] (float32) of a matrix's bytes."""
    b = np.asarray(data, dtype=np.uint8).reshape(-1)
    assert b.size == rows * cols + 4 * rows
    codes = b[:rows * cols].reshape(rows, cols)
    scales = b[rows * cols:].copy().view("<f4")
    return codes, scales


def decode_matrix(data, rows, cols):
    """FP8 bytes of a [rows, cols] matrix -> float64 [rows, cols] (exact)."""
    codes, scales = split(data, rows, cols)
    return scales.astype(np.float64)[:, None] * decode_codes(codes)
