"""GPU parity of the Q4_K kernels and of prefix acceptance against the oracle.

Q4_K decode is bit-exact (every block of every drafter matrix shape at full
size); the GEMM matches the oracle's float64 product to the bf16 rounding of
its output.
"""
import sys

import numpy as np
import pytest
import torch

from block_diffusion_draft_amd import binding, synth
from oracle import q4k as oq4k
from oracle.bf16 import bf16_to_f64
from oracle.verify import verify_prefix

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


@pytest.mark.parametrize("name,N,K", synth.GEMM_SHAPES)
def test_q4k_dequantize_bit_exact_full_matrix(name, N, K):
    say(f"[q4k_dequantize] {name} {N}x{K}")
    w, _ = synth.gemm_inputs(name, N, K)
    wd = dev_u8(w)
    rows_per = max(1, (1 << 24) // K)
    for r0 in range(0, N, rows_per):
        r1 = min(N, r0 + rows_per)
        nb = (r1 - r0) * (K // 256)
        out = torch.empty(nb * 256, dtype=torch.float32, device="cuda")
        seg = wd[r0 * (K // 256) * 144: r1 * (K // 256) * 144]
        binding.q4k_dequantize(seg, out)
        got = out.cpu().numpy()
        ref = oq4k.decode_matrix(w[r0 * (K // 256) * 144: r1 * (K // 256) * 144], r1 - r0, K)
        assert np.array_equal(got.view(np.uint32),
                              ref.astype(np.float32).reshape(-1).view(np.uint32)), (name, r0)


def tiled_reference(w, N, K):
    """The tiled Q4_K layout written out from its definition (a byte permutation of
    the row-major blocks: 16 headers, then per half h the 16-byte slots 16 g + r
    holding bytes 8 g .. 8 g + 7 of chunks 2 h and 2 h + 1)."""
    KB = K // 256
    blk = w.reshape(N // 16, 16, KB, 144).transpose(0, 2, 1, 3)       # [t][kb][r][144]
    hdr = blk[..., :16].reshape(N // 16, KB, 256)
    q = blk[..., 16:].reshape(N // 16, KB, 16, 4, 4, 8)                 # [t][kb][r][c][g][8]
    halves = []
    for h in range(2):
        pair = np.concatenate([q[:, :, :, 2 * h], q[:, :, :, 2 * h + 1]], axis=-1)  # [t][kb][r][g][16]
        halves.append(pair.transpose(0, 1, 3, 2, 4).reshape(N // 16, KB, 1024))   # slot 16 g + r
    return np.concatenate([hdr] + halves, axis=-1).reshape(-1)


def dev_tiled(w, N, K):
    src = dev_u8(w)
    dst = torch.empty_like(src)
    binding.q4k_to_tiled(src, dst, N, K)
    return dst


@pytest.mark.parametrize("N,K", [(16, 256), (48, 768), (5120, 4096)])
def test_q4k_to_tiled_byte_exact(N, K):
    say(f"[q4k_to_tiled] {N}x{K}")
    w = synth.q4k_normal(7, "tiled", N, K, 0.02)
    got = dev_tiled(w, N, K).cpu().numpy()
    assert np.array_equal(got, tiled_reference(w, N, K))


def gemm_check(w, x, N, K, M):
    """Up to 16 rows with K / 256 a multiple of 4 the streaming kernel (exact products
    of the decoded weights), else the many-row GEMM (each weight as two bf16 terms,
    within 2^-18 of it).  The bound is the output's bf16 rounding plus fp32
    accumulation; it holds no term for rounding the weights."""
    wd = dev_tiled(w, N, K)
    xd = dev_bf16(x)
    y = torch.empty((M, N), dtype=torch.int16, device="cuda")
    ws = torch.empty(binding.q4k_gemm_tiled_workspace_bytes(M, N, K), dtype=torch.uint8,
                     device="cuda")
    binding.q4k_gemm_tiled(wd, xd, y, ws)
    # the row-major entry point (GGUF byte order) regroups in its workspace and must
    # give the same bits
    y2 = torch.empty_like(y)
    ws2 = torch.empty(binding.q4k_gemm_workspace_bytes(M, N, K), dtype=torch.uint8,
                      device="cuda")
    binding.q4k_gemm(dev_u8(w), xd, y2, ws2)
    assert torch.equal(y, y2)
    got = bf16_to_f64(y.cpu().numpy().view(np.uint16))
    xf = bf16_to_f64(x)
    W = oq4k.decode_matrix(w, N, K)
    ref = xf @ W.T
    # output rounded to bf16 (<= 2^-9 relative) plus fp32 accumulation
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-5 * np.sqrt(np.mean(ref ** 2))
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    assert np.all(err <= bound), (float((err / np.maximum(bound, 1e-30)).max()), rel)
    return rel


@pytest.mark.parametrize("name,N,K", synth.GEMM_SHAPES)
def test_q4k_gemm_drafter_shapes_m8(name, N, K):
    say(f"[q4k_gemm] {name} M=8 {N}x{K}")
    w, x = synth.gemm_inputs(name, N, K, M=8)
    rel = gemm_check(w, x, N, K, 8)
    assert rel < 3e-3


@pytest.mark.parametrize("M", [1, 3, 16, 17, 40, 64, 65, 128])
def test_q4k_gemm_row_counts(M):
    """Ragged row counts across MFMA row tiles and row groups."""
    N, K = 272, 1280
    say(f"[q4k_gemm] M={M} {N}x{K}")
    w = synth.q4k_normal(5, "rows", N, K, 0.02)
    x = synth.normal_bf16(5, "rows.x", (M, K), 1.0)
    gemm_check(w, x, N, K, M)


@pytest.mark.parametrize("M,N,K", [(1, 16, 1024), (8, 16, 2048), (3, 48, 1024), (16, 48, 2048),
                                   (8, 272, 2048), (16, 272, 4096)])
def test_q4k_gemm_stream_few_tiles(M, N, K):
    """The streaming kernel (up to 16 rows, K a multiple of 1024) where a split has fewer
    column tiles than its workgroup has waves (1, 3 and 17 tiles for 8 waves): the waves
    without a tile only run their clamped loads, the others their runs."""
    say(f"[q4k_gemm stream] M={M} {N}x{K}")
    w = synth.q4k_normal(9, "few", N, K, 0.02)
    x = synth.normal_bf16(9, "few.x", (M, K), 1.0)
    gemm_check(w, x, N, K, M)


@pytest.mark.parametrize("M,N,K", [(160, 4096, 4096), (256, 8704, 5120), (136, 34816, 4096),
                                   (512, 34816, 2048), (1000, 8704, 4096)])
def test_q4k_gemm_schedules(M, N, K):
    """Many-row GEMM schedules: 16 and 34 tiles of 256 rows run as one round of K splits
    (13 and 7 splits); 136 tiles (ragged rows) as stream-K, each CU one equal range of
    (tile, K stage) units, the pieces of a tile in their own partial slots (3), unused
    slots zeroed; 2 and 4 M tiles (the last ragged) as grouped stream-K, ranges of
    (group of 16 / 4 weight slabs, K stage) units each worked by one workgroup per (M
    tile, slab of the group), some slabs of the last group past the matrix (2 and 3
    slots)."""
    say(f"[q4k_gemm schedules] M={M} {N}x{K}")
    w = synth.q4k_normal(8, "sk", N, K, 0.02)
    x = synth.normal_bf16(8, "sk.x", (M, K), 1.0)
    gemm_check(w, x, N, K, M)


@pytest.mark.parametrize("M,N,K", [(40, 272, 256), (17, 272, 512), (256, 272, 768),
                                   (40, 16640, 1024)])
def test_q4k_gemm_many_rows_short_k(M, N, K):
    """Many-row GEMM over 1-4 super-blocks: its raw weight bytes go through two LDS
    slots of half a super-block each, requested four 32-deep stages ahead, so pieces of
    8, 16 and 24 stages request halves past their end (clamped to the last one); the
    last shape runs as a grid of 3 K splits of 5, 5 and 6 64-deep units, the second
    starting in the middle of a half super-block."""
    say(f"[q4k_gemm many rows short K] M={M} {N}x{K}")
    w = synth.q4k_normal(10, "shortk", N, K, 0.02)
    x = synth.normal_bf16(10, "shortk.x", (M, K), 1.0)
    gemm_check(w, x, N, K, M)


def test_q4k_gemm_one_block_edge():
    """Smallest shape: one super-block, one column tile."""
    N, K, M = 16, 256, 2
    w = synth.q4k_normal(6, "edge", N, K, 0.02)
    x = synth.normal_bf16(6, "edge.x", (M, K), 1.0)
    gemm_check(w, x, N, K, M)


def test_verify_prefix_all_lengths_and_random():
    rng = np.random.default_rng(0)
    B, n = 64, 7
    draft = rng.integers(0, 248320, size=(B, n)).astype(np.int32)
    tgt = rng.integers(0, 248320, size=(B, n + 1)).astype(np.int32)
    for b in range(B):
        k = b % (n + 1)
        tgt[b, :k] = draft[b, :k]
        if k < n:
            tgt[b, k] = (draft[b, k] + 1) % 248320
    acc = torch.empty(B, dtype=torch.int32, device="cuda")
    out = torch.empty((B, n + 1), dtype=torch.int32, device="cuda")
    binding.verify_prefix(torch.from_numpy(draft).cuda(), torch.from_numpy(tgt).cuda(), acc, out)
    ra, ro = verify_prefix(draft, tgt)
    assert np.array_equal(acc.cpu().numpy(), ra)
    assert np.array_equal(out.cpu().numpy(), ro)
