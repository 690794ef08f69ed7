"""Q8_0 block decode (test infrastructure only).

Source: Mindket kit page "Qwen3.8-27B-DFlash2-GGUF by z-lab", the draft-file table
(a Q8_0 draft file of 2.0 GB beside the Q4_K_M and BF16 ones) and "Good to know"
(its acceptance length).  The pages name the format, not its bytes; the reading
taken is the GGUF Q8_0 block:

    34 bytes per 32 consecutive weights of a row:
        bytes 0..1   d  (fp16, little endian)
        bytes 2..33  q  (32 signed bytes, weight i of the block at byte 2 + i)
    w = d * q.

A matrix [N rows][K cols] (y = x . W^T, K along the input) is stored as N rows of
K/32 consecutive blocks.
"""
import numpy as np

BLOCK_BYTES = 34
BLOCK_WEIGHTS = 32


def decode_blocks(blocks):
    """uint8 blocks [..., 34] -> float64 weights [..., 32]."""
    b = np.asarray(blocks, dtype=np.uint8)
    assert b.shape[-1] == BLOCK_BYTES
    d = b[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
    q = b[..., 2:].view(np.int8).astype(np.float64)
    return d[..., None] * q


def decode_matrix(data, rows, cols):
    """Q8_0 bytes of a [rows, cols] matrix -> float64 [rows, cols]."""
    assert cols % BLOCK_WEIGHTS == 0
    blocks = np.asarray(data, dtype=np.uint8).reshape(rows, cols // BLOCK_WEIGHTS, BLOCK_BYTES)
    return decode_blocks(blocks).reshape(rows, cols)
