"""Pins of the oracle's Q4_K decode and of the host Q4_K packer (CPU only)."""
import os

import numpy as np
import pytest

from oracle import q4k

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "q4k_block_handmade.txt")


def load_golden():
    fields = {}
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        k, *v = line.split()
        fields[k] = v
    head = bytes.fromhex(fields["hex"][0])
    block = np.frombuffer(head + bytes(range(128)), dtype=np.uint8)
    return (block, float(fields["d"][0]), float(fields["dmin"][0]),
            [int(x) for x in fields["sc"]], [int(x) for x in fields["m"]])


def test_handmade_block_fields():
    block, d, dmin, sc, m = load_golden()
    dd, dm, s, mm, q = q4k.block_fields(block)
    assert dd == d and dm == dmin
    assert list(s) == sc and list(mm) == m
    for i in range(256):
        c, r = divmod(i, 64)
        want = (r & 15) if r < 32 else 2 * c + ((r - 32) >> 4)
        assert q[i] == want, i


def test_handmade_block_weights():
    block, d, dmin, sc, m = load_golden()
    w = q4k.decode_blocks(block)
    for i in range(256):
        c, r = divmod(i, 64)
        qi = (r & 15) if r < 32 else 2 * c + ((r - 32) >> 4)
        j = i // 32
        assert w[i] == d * sc[j] * qi - dmin * m[j], i


def test_unit_scale_ramp():
    """d = 1, dmin = 0, every sc = 1, q_i = i % 16  ->  w_i = i % 16."""
    head = bytes.fromhex("003c0000") + bytes([1, 1, 1, 1, 0, 0, 0, 0, 1, 1, 1, 1])
    qs = bytearray(128)
    for i in range(256):
        c, r = divmod(i, 64)
        if r < 32:
            qs[32 * c + r] |= i % 16
        else:
            qs[32 * c + r - 32] |= (i % 16) << 4
    w = q4k.decode_blocks(np.frombuffer(head + bytes(qs), dtype=np.uint8))
    assert np.array_equal(w, np.arange(256) % 16)


@pytest.mark.parametrize("j", range(8))
def test_every_six_bit_field(j):
    """Sweep sc_j and m_j over 0..63 (the split high bits of j >= 4 included)
    with q = 1 everywhere, d = 1, dmin = 1: every weight of sub-block j equals
    sc_j - m_j and the other sub-blocks stay at 0."""
    for v in range(64):
        s = [0] * 12
        sc = [0] * 8
        mm = [0] * 8
        sc[j] = v
        mm[j] = 63 - v
        for k in range(4):
            s[k] = (sc[k] & 63) | ((sc[k + 4] >> 4) << 6)
            s[k + 4] = (mm[k] & 63) | ((mm[k + 4] >> 4) << 6)
            s[k + 8] = (sc[k + 4] & 15) | ((mm[k + 4] & 15) << 4)
        head = bytes.fromhex("003c003c") + bytes(s)
        w = q4k.decode_blocks(np.frombuffer(head + bytes([0x11] * 128), dtype=np.uint8))
        exp = np.zeros(256)
        exp[32 * j:32 * j + 32] = v - (63 - v)
        assert np.array_equal(w, exp), (j, v)


def test_matrix_layout_rows_of_blocks():
    """A [2, 512] matrix is 2 rows x 2 blocks; row r block b decodes to cols 256b.."""
    blocks = []
    for r in range(2):
        for b in range(2):
            val = 1 + 2 * r + b       # constant q per block, d = 1, sc = 1, dmin = 0
            head = bytes.fromhex("003c0000") + bytes([1, 1, 1, 1, 0, 0, 0, 0, 1, 1, 1, 1])
            blocks.append(head + bytes([val | (val << 4)] * 128))
    W = q4k.decode_matrix(b"".join(blocks), 2, 512)
    assert np.array_equal(W[0, :256], np.full(256, 1.0))
    assert np.array_equal(W[0, 256:], np.full(256, 2.0))
    assert np.array_equal(W[1, :256], np.full(256, 3.0))
    assert np.array_equal(W[1, 256:], np.full(256, 4.0))


def test_packer_round_trip_error_matches_pages():
    """The FastFlowLM card ("Weights" row) reports about 0.07 relative L2 per
    matrix for its Q4_K weights; the host packer on N(0, 0.02) matrices must land
    in the same place (band [0.06, 0.085])."""
    from block_diffusion_draft_amd import synth
    for seed, (rows, cols) in [(1, (512, 4096)), (2, (256, 5120))]:
        w = synth.normal_f32(seed, "roundtrip", (rows, cols), 0.02)
        deq = q4k.decode_matrix(synth.q4k_pack(w), rows, cols)
        rel = np.linalg.norm(deq - w) / np.linalg.norm(w)
        assert 0.06 <= rel <= 0.085, rel


def test_packer_fields_in_range_and_codes_consistent():
    """Decoded blocks of the packer reproduce the input's per-block mean to
    within one quantisation step (catches a sign or offset error in dmin*m)."""
    from block_diffusion_draft_amd import synth
    w = synth.normal_f32(7, "fields", (64, 1024), 0.02)
    b = synth.q4k_pack(w).reshape(64, 4, 144)
    d, dmin, sc, m, q = q4k.block_fields(b)
    assert (sc >= 0).all() and (sc <= 63).all() and (m >= 0).all() and (m <= 63).all()
    assert (q >= 0).all() and (q <= 15).all()
    deq = q4k.decode_blocks(b).reshape(64, 1024)
    step = (d[..., None] * sc).max()
    assert np.abs(deq.reshape(64, 4, 256).mean(-1) - w.reshape(64, 4, 256).mean(-1)).max() < step
