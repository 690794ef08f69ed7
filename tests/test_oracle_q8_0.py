"""Pins of the Q8_0 decode oracle.

Mindket kit page "Qwen3.8-27B-DFlash2-GGUF by z-lab": the draft ships as Q4_K_M, Q8_0
and BF16 files (draft-file table, 1.1 / 2.0 / 3.8 GB).  Pinned by a block written by
hand, a closed-form ramp, the byte layout of a matrix, the quantizer's error bound,
and the file sizes the page states against the stated parameter count.
"""
import os

import numpy as np

from block_diffusion_draft_amd import synth
from oracle import budget, q8_0

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "q8_0_block_handmade.txt")


def read_golden():
    hexs, w = "", []
    for line in open(GOLDEN):
        if line.startswith("hex"):
            hexs = line.split(None, 1)[1].replace(" ", "").strip()
        elif line.startswith("w "):
            w += [float(v) for v in line.split()[1:]]
    return np.frombuffer(bytes.fromhex(hexs), dtype=np.uint8), np.array(w)


def test_handmade_block():
    blk, want = read_golden()
    assert blk.size == q8_0.BLOCK_BYTES and want.size == 32
    assert np.array_equal(q8_0.decode_blocks(blk), want)


def test_power_of_two_ramp():
    # d = 2^-7 (fp16 0x2000): weight = q / 128 for every signed byte value
    q = np.arange(-128, 128, dtype=np.int32)
    blocks = np.zeros((8, 34), dtype=np.uint8)
    blocks[:, 0], blocks[:, 1] = 0x00, 0x20
    blocks[:, 2:] = (q.reshape(8, 32) & 0xFF).astype(np.uint8)
    assert np.array_equal(q8_0.decode_blocks(blocks).reshape(-1), q / 128.0)


def test_matrix_layout():
    rows, cols = 3, 96
    data = np.zeros(rows * (cols // 32) * 34, dtype=np.uint8)
    data.reshape(rows, cols // 32, 34)[:, :, 1] = 0x3C          # d = 1.0 everywhere
    r, b, i = 2, 1, 17
    data[(r * (cols // 32) + b) * 34 + 2 + i] = 0xF9           # q = -7 at weight 32 b + i
    w = q8_0.decode_matrix(data, rows, cols)
    want = np.zeros((rows, cols))
    want[r, 32 * b + i] = -7.0
    assert np.array_equal(w, want)


def test_quantizer_round_trip_bound():
    x = synth.normal_f32(2, "q8.rt", (64, 512), 0.02)
    data = synth.q8_0_pack(x)
    w = q8_0.decode_matrix(data, 64, 512)
    d = data.reshape(64, 16, 34)[:, :, :2].copy().view(np.float16)[..., 0].astype(np.float64)
    err = np.abs(w - x.astype(np.float64)).reshape(64, 16, 32)
    assert (err <= d[..., None] / 2 * (1 + 1e-9)).all()         # round to nearest code
    rel = np.linalg.norm(w - x) / np.linalg.norm(x)
    assert 0.003 < rel < 0.008, rel                               # about 1 / (127 sqrt 12) * 2.2


def test_file_sizes_match_the_stated_parameter_count():
    # 34 bytes per 32 weights: the stated 1,924,404,480 parameters in Q8_0 are the
    # 2.0 GB draft file; at 2 bytes each, the 3.8 GB BF16 file
    n = budget.STATED_PARAMS
    assert abs(n * 34 / 32 / 1e9 - 2.0) < 0.05
    assert abs(n * 2 / 1e9 - 3.8) < 0.05
