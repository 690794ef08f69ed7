"""Q4_K super-block decode (test infrastructure only).

Source: FastFlowLM card "Qwen3.8-27B-DFlash2-NPU2", spec table, "Weights" row:
the fc, q/k/v/o and MLP matrices are stored in Q4_K.  The structure used here is
the one stated for the draft's quantised weights: 256-weight super-blocks, each
split into 8 sub-blocks of 32 weights, with 6-bit per-sub-block scales and mins
and an fp16 super-block scale d and min-scale dmin.  Each weight is

    w = d * sc_j * q - dmin * m_j ,   j = sub-block of the weight, q in 0..15.

Byte layout of one 144-byte block (the common GGUF Q4_K packing; the pages give
the structure, not the bytes -- reading recorded in the design notes):
    bytes   0..1   d     (fp16, little endian)
    bytes   2..3   dmin  (fp16, little endian)
    bytes   4..15  scales[12]:
        j < 4 : sc_j = scales[j] & 63          m_j = scales[j+4] & 63
        j >= 4: sc_j = (scales[j+4] & 15) | ((scales[j-4] >> 6) << 4)
                m_j  = (scales[j+4] >> 4) | ((scales[j]   >> 6) << 4)
    bytes  16..143 qs[128]: 32-byte chunk c covers weights 64c .. 64c+63;
        weight 64c + i    (i < 32) is the low  nibble of qs[32c + i],
        weight 64c + 32+i (i < 32) is the high nibble of qs[32c + i].

A matrix [N rows][K cols] (y = x . W^T, K along the input) is stored as
N rows of K/256 consecutive blocks.
"""
import numpy as np

BLOCK_BYTES = 144
BLOCK_WEIGHTS = 256


def block_fields(blocks):
    """Split uint8 blocks [..., 144] into (d, dmin, sc[...,8], m[...,8], q[...,256]).

    d, dmin are float64; sc, m, q are integer arrays.
    """
    b = np.asarray(blocks, dtype=np.uint8)
    assert b.shape[-1] == BLOCK_BYTES
    lead = b.shape[:-1]
    d = b[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
    dmin = b[..., 2:4].copy().view(np.float16)[..., 0].astype(np.float64)
    s = b[..., 4:16].astype(np.int64)
    sc = np.empty(lead + (8,), dtype=np.int64)
    m = np.empty(lead + (8,), dtype=np.int64)
    for j in range(8):
        if j < 4:
            sc[..., j] = s[..., j] & 63
            m[..., j] = s[..., j + 4] & 63
        else:
            sc[..., j] = (s[..., j + 4] & 15) | ((s[..., j - 4] >> 6) << 4)
            m[..., j] = (s[..., j + 4] >> 4) | ((s[..., j] >> 6) << 4)
    qs = b[..., 16:144].reshape(lead + (4, 32))
    lo = qs & 15
    hi = qs >> 4
    q = np.stack([lo, hi], axis=-2).reshape(lead + (256,)).astype(np.int64)
    return d, dmin, sc, m, q


def decode_blocks(blocks):
    """uint8 blocks [..., 144] -> float64 weights [..., 256]."""
    d, dmin, sc, m, q = block_fields(blocks)
    lead = q.shape[:-1]
    q = q.reshape(lead + (8, 32)).astype(np.float64)
    w = (d[..., None, None] * sc[..., :, None].astype(np.float64)) * q \
        - (dmin[..., None] * m.astype(np.float64))[..., :, None]
    return w.reshape(lead + (256,))


def decode_matrix(raw, rows, cols):
    """Q4_K bytes of a [rows, cols] matrix -> float64 [rows, cols]."""
    assert cols % BLOCK_WEIGHTS == 0
    nb = cols // BLOCK_WEIGHTS
    if isinstance(raw, (bytes, bytearray, memoryview)):
        b = np.frombuffer(raw, dtype=np.uint8)
    else:
        b = np.ascontiguousarray(raw, dtype=np.uint8).reshape(-1)
    assert b.size == rows * nb * BLOCK_BYTES, (b.size, rows, cols)
    b = b.reshape(rows, nb, BLOCK_BYTES)
    out = np.empty((rows, cols), dtype=np.float64)
    step = max(1, (1 << 22) // cols)            # bounded temporaries
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        out[r0:r1] = decode_blocks(b[r0:r1]).reshape(r1 - r0, cols)
    return out


def matrix_bytes(rows, cols):
    return rows * (cols // BLOCK_WEIGHTS) * BLOCK_BYTES
