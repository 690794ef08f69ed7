"""GPU parity of the Q8_0 weight path against the oracle.

Mindket kit page "Qwen3.8-27B-DFlash2-GGUF by z-lab", draft-file table: the draft
also ships as a Q8_0 file (GGUF Q8_0 blocks: fp16 scale, 32 signed bytes).  Decode is
bit-exact; the tiled layout byte-exact against its definition; the 16-row streaming
GEMM matches the float64 product to the bf16 rounding of its output (its products
d q are exact), and so does the many-row MFMA GEMM (more rows, or K not a multiple of
1024), whose weights enter as two bf16 terms within 2^-18 of d q; whole draft steps
with Q8_0 weights meet the step's parity bars.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

from block_diffusion_draft_amd import binding, runner, synth
from oracle import q8_0 as oq8
from oracle.bf16 import bf16_to_f64
from tests import parity
from tests.test_gpu_step import check_verify, full_check

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def tiled_reference(w, N, K):
    """The tiled Q8_0 layout written out from its definition: per (16-row tile, 256-wide
    K-group) the rows' 8 block scales, then per block pair p the 16-byte slots 16 h + r
    holding bytes 8 h .. 8 h + 7 of blocks 2 p and 2 p + 1 of row r."""
    G = K // 256
    blk = w.reshape(N // 16, 16, G, 8, 34).transpose(0, 2, 1, 3, 4)   # [t][g][r][b][34]
    sc = blk[..., :2].reshape(N // 16, G, 256)
    q = blk[..., 2:].reshape(N // 16, G, 16, 4, 2, 4, 8)              # [t][g][r][p][b2][h][8]
    q = q.transpose(0, 1, 3, 5, 2, 4, 6).reshape(N // 16, G, 4096)    # [t][g][p][h][r][b2][8]
    return np.concatenate([sc, q], axis=-1).reshape(-1)


def dev_tiled(w, N, K):
    src = dev_u8(w)
    dst = torch.empty_like(src)
    binding.q8_0_to_tiled(src, dst, N, K)
    return dst


@pytest.mark.parametrize("N,K", [(16, 256), (48, 768), (5120, 4096)])
def test_q8_0_to_tiled_byte_exact(N, K):
    say(f"[q8_0_to_tiled] {N}x{K}")
    w = synth.q8_0_normal(7, "q8.tiled", N, K, 0.02)
    got = dev_tiled(w, N, K).cpu().numpy()
    assert np.array_equal(got, tiled_reference(w, N, K))


@pytest.mark.parametrize("N,K", [(4096, 5120), (1024, 5120), (3, 96)])
def test_q8_0_dequantize_bit_exact(N, K):
    say(f"[q8_0_dequantize] {N}x{K}")
    w = synth.q8_0_normal(8, "q8.deq", N, K, 0.02)
    out = torch.empty(N * K, dtype=torch.float32, device="cuda")
    binding.q8_0_dequantize(dev_u8(w), out)
    ref = oq8.decode_matrix(w, N, K).astype(np.float32).reshape(-1)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def gemm_check(w, x, N, K, M):
    wd = dev_tiled(w, N, K)
    y = torch.empty((M, N), dtype=torch.int16, device="cuda")
    ws = torch.empty(binding.q8_0_gemm_tiled_workspace_bytes(M, N, K), dtype=torch.uint8,
                     device="cuda")
    binding.q8_0_gemm_tiled(wd, dev_bf16(x), y, ws)
    # the row-major entry point regroups in its workspace and must give the same bits
    y2 = torch.empty_like(y)
    ws2 = torch.empty(binding.q8_0_gemm_workspace_bytes(M, N, K), dtype=torch.uint8,
                      device="cuda")
    binding.q8_0_gemm(dev_u8(w), dev_bf16(x), y2, ws2)
    assert torch.equal(y, y2)
    got = bf16_to_f64(y.cpu().numpy().view(np.uint16))
    xf = bf16_to_f64(x)
    W = oq8.decode_matrix(w, N, K)
    ref = xf @ W.T
    err = np.abs(got - ref)
    # output rounded to bf16 (<= 2^-9 relative) plus fp32 accumulation
    bound = 2.0 ** -8 * np.abs(ref) + 1e-5 * np.sqrt(np.mean(ref ** 2))
    assert np.all(err <= bound), float((err / np.maximum(bound, 1e-30)).max())
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


@pytest.mark.parametrize("name,N,K", synth.GEMM_SHAPES)
def test_q8_0_gemm_drafter_shapes_m8(name, N, K):
    say(f"[q8_0_gemm] {name} M=8 {N}x{K}")
    w = synth.q8_0_normal(synth.GEMM_SEED, f"gemm.{name}", N, K, 0.02)
    x = synth.normal_bf16(synth.GEMM_SEED, f"gemm.{name}.x", (8, K), 1.0)
    rel = gemm_check(w, x, N, K, 8)
    assert rel < 3e-3


@pytest.mark.parametrize("M,K", [(1, 2048), (3, 2048), (16, 2048), (1, 1280), (16, 1280),
                                 (17, 1280), (40, 2048), (128, 1280), (300, 2048)])
def test_q8_0_gemm_row_counts(M, K):
    """Ragged row counts: up to 16 rows with K % 1024 == 0 the streaming kernel, the
    rest the tiled kernel (ragged row and column tiles)."""
    N = 272
    say(f"[q8_0_gemm] M={M} {N}x{K}")
    w = synth.q8_0_normal(5, "q8.rows", N, K, 0.02)
    x = synth.normal_bf16(5, "q8.rows.x", (M, K), 1.0)
    gemm_check(w, x, N, K, M)


@pytest.mark.parametrize("M,N,K", [(160, 4096, 4096), (256, 8704, 5120), (136, 34816, 4096)])
def test_q8_0_gemm_schedules(M, N, K):
    """Many-row GEMM schedules: one round of K splits (16 and 34 tiles), stream-K (136)."""
    say(f"[q8_0_gemm schedules] M={M} {N}x{K}")
    w = synth.q8_0_normal(8, "q8.sk", N, K, 0.02)
    x = synth.normal_bf16(8, "q8.sk.x", (M, K), 1.0)
    gemm_check(w, x, N, K, M)


@pytest.mark.parametrize("shape,batch", [("mid", 1), ("mid", 2), ("mid", 16), ("tiny", 2)])
def test_small_step_q8_0(shape, batch):
    """Whole draft steps with Q8_0 weights: a 2-layer drafter whose products all take the
    streaming kernel (1 sequence) or the tiled one (2 sequences: 32 MLP rows; 16
    sequences: 256 MLP rows over two row tiles), and the tiny drafter (K = 256 and 1280:
    the tiled kernel)."""
    s = dataclasses.replace(synth.MID if shape == "mid" else synth.TINY, weight_fmt="q8_0")
    wl = dataclasses.replace(synth.WORKLOADS["tiny"], shape=s, batch=batch, ctx_len=96,
                             seed=40 + batch)
    say(f"[step q8_0] {shape} batch {batch}")
    bufs = runner.StepBuffers(wl)
    bufs.step()
    torch.cuda.synchronize()
    ref = parity.run_oracle(wl, bufs.host_W, bufs.inputs)
    g = full_check(wl, bufs, ref)
    check_verify(bufs, g)


@pytest.mark.timeout(900)
def test_full_step_b1_q8_0_parity():
    """The pages' draft shape with Q8_0 drafter weights, one sequence, 4096 cached rows."""
    wl = synth.WORKLOADS["full_b1_q8_0"]
    say(f"[step] {wl.name}: generating inputs")
    bufs = runner.StepBuffers(wl)
    say("  running GPU step")
    bufs.step()
    torch.cuda.synchronize()
    say("  running oracle")
    ref = parity.run_oracle(wl, bufs.host_W, bufs.inputs)
    g = full_check(wl, bufs, ref)
    check_verify(bufs, g)
