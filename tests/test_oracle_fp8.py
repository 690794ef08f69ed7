"""Pins of the FP8 decode oracle.

aiqre model page "Qwen3.8-27B-DFlash2", "Memory": an fp8 weight format at one byte per
parameter, 1.8 GiB for the drafter.  Pinned by a matrix written by hand, every code
against the E4M3 conversion of a library (torch.float8_e4m3fn), the byte layout of a
matrix, the host quantizer's rounding bound, and the page's memory figure against the
stated parameter count.
"""
import math
import os

import numpy as np
import torch

from block_diffusion_draft_amd import synth
from oracle import budget, fp8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fp8_e4m3_handmade.txt")


def read_golden():
    hexs, w = "", []
    for line in open(GOLDEN):
        if line.startswith("hex"):
            hexs = line.split(None, 1)[1].replace(" ", "").strip()
        elif line.startswith("w "):
            w += [float(v) for v in line.split()[1:]]
    return np.frombuffer(bytes.fromhex(hexs), dtype=np.uint8), np.array(w).reshape(2, 8)


def test_handmade_matrix():
    data, want = read_golden()
    assert data.size == 2 * 8 + 2 * 4
    got = fp8.decode_matrix(data, 2, 8)
    assert np.array_equal(got, want)
    assert np.signbit(got[1, 0]) and not np.signbit(got[0, 0])     # -0 and +0


def test_every_code_against_the_library_conversion():
    codes = np.arange(256, dtype=np.uint8)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = fp8.decode_codes(codes)
    nan = np.isnan(lib)
    assert np.array_equal(nan, np.isnan(ours))
    assert set(np.flatnonzero(nan)) == {0x7F, 0xFF}
    assert np.array_equal(lib[~nan], ours[~nan])
    assert np.array_equal(np.signbit(lib[~nan]), np.signbit(ours[~nan]))


def test_code_order_and_range():
    v = fp8.decode_codes(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(v) > 0)                   # positive codes increase strictly
    assert v[1] == 2.0 ** -9 and v[-1] == 448.0
    neg = fp8.decode_codes(np.arange(0x80, 0xFF, dtype=np.uint8))
    assert np.array_equal(neg, -v)


def test_matrix_layout():
    rows, cols = 3, 64
    data = np.zeros(synth.fp8_bytes(rows, cols), dtype=np.uint8)
    data[rows * cols:] = np.array([1.0, 2.0, 0.25], dtype="<f4").view(np.uint8)
    r, c = 2, 37
    data[r * cols + c] = 0x3C                       # 1.5 at (2, 37)
    w = fp8.decode_matrix(data, rows, cols)
    want = np.zeros((rows, cols))
    want[r, c] = 1.5 * 0.25
    assert np.array_equal(w, want)
    data[rows * cols + 4 * 2: rows * cols + 4 * 3] = np.array([4.0], dtype="<f4").view(np.uint8)
    assert fp8.decode_matrix(data, rows, cols)[r, c] == 6.0


def test_quantizer_round_trip_bound():
    x = synth.normal_f32(3, "fp8.rt", (64, 512), 0.02)
    data = synth.fp8_pack(x)
    codes, scales = fp8.split(data, 64, 512)
    s = scales.astype(np.float64)
    amax = np.abs(x.astype(np.float64)).max(axis=1)
    assert np.allclose(s, amax / 448.0, rtol=2.0 ** -23)
    w = fp8.decode_matrix(data, 64, 512)
    # nearest E4M3 value: within half the spacing at that magnitude (2^(e-3) for a
    # normal of exponent e, 2^-9 below 2^-6), in units of the row scale
    a = np.abs(x.astype(np.float64)) / s[:, None]
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    half = 2.0 ** (e - 3) / 2
    err = np.abs(w - x.astype(np.float64)) / s[:, None]
    assert (err <= half * (1 + 1e-9)).all()
    rel = np.linalg.norm(w - x) / np.linalg.norm(x)
    assert 0.01 < rel < 0.04, rel                   # 3 mantissa bits: about 2^-4 / sqrt(3)


def test_memory_figure_matches_the_stated_parameter_count():
    # one byte per parameter: 1,924,404,480 B = 1.79 GiB, the page's "1.8 GiB"; the
    # per-row scales add 4 bytes per output row of each linear matrix (< 0.1 MiB here)
    n = budget.STATED_PARAMS
    assert round(n / 2 ** 30, 1) == 1.8
    rows = 5120 + 5 * (4096 + 2 * 1024 + 5120 + 2 * 17408 + 5120)
    assert 4 * rows < 2 ** 20
    assert math.isclose(n * 2 / 2 ** 30, 3.6, abs_tol=0.05)     # the bf16 row
