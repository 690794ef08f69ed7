"""GPU parity of the FP8 weight path against the oracle.

aiqre model page "Qwen3.8-27B-DFlash2", "Memory": an fp8 weight format at one byte per
parameter (read as OCP E4M3 codes with one fp32 scale per output row).  Decode is
bit-exact on every one of the 256 codes (NaN codes give NaN) and on packed matrices;
the tiled layout is byte-exact against its definition; the 16-row streaming GEMM and
the many-row MFMA GEMM match the float64 product to the bf16 rounding of their output
(every E4M3 value is exact in bf16, the row scale multiplies the fp32 sum), on packed
weights and on arbitrary codes and scales; whole draft steps with FP8 weights meet the
step's parity bars.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

from block_diffusion_draft_amd import binding, runner, synth
from oracle import fp8 as of8
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


def make_matrix(codes, scales):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    return np.concatenate([codes.reshape(-1), np.asarray(scales, dtype="<f4").view(np.uint8)])


def tiled_reference(w, N, K):
    """The tiled FP8 layout written out from its definition: per (16-row tile, 256-wide
    K-group) and pair p the 16-byte slots 16 h + r holding codes 64 p + 8 h .. + 7 of row
    r, then its codes 64 p + 32 + 8 h .. + 7; then the row scales unchanged."""
    G = K // 256
    c = w[:N * K].reshape(N // 16, 16, G, 4, 2, 4, 8)          # [t][r][g][p][b2][h][8]
    c = c.transpose(0, 2, 3, 5, 1, 4, 6).reshape(-1)           # [t][g][p][h][r][b2][8]
    return np.concatenate([c, w[N * K:]])


def dev_tiled(w, N, K):
    src = dev_u8(w)
    dst = torch.empty_like(src)
    binding.fp8_to_tiled(src, dst, N, K)
    return dst


def test_fp8_dequantize_every_code():
    """All 256 codes in every row, rows with scales of both signs, powers of two and
    others; NaN codes decode to NaN, every other value bit-exact."""
    N, K = 16, 256
    rng = np.random.default_rng(11)
    codes = np.stack([rng.permutation(256) for _ in range(N)]).astype(np.uint8)
    scales = np.array([1.0, 2.0 ** -10, 3.7, -0.25, 448.0, 1e-3, -7.5, 2.0 ** 20,
                       0.02 / 448, 1.5, -1.0, 0.75, 123.0, 2.0 ** -30, 5.0, 0.1], dtype=np.float32)
    w = make_matrix(codes, scales)
    out = torch.empty((N, K), dtype=torch.float32, device="cuda")
    binding.fp8_dequantize(dev_u8(w), out)
    got = out.cpu().numpy()
    ref = of8.decode_matrix(w, N, K).astype(np.float32)
    nan = np.isnan(ref)
    assert nan.sum() == 2 * N
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


@pytest.mark.parametrize("N,K", [(4096, 5120), (48, 768)])
def test_fp8_dequantize_packed(N, K):
    say(f"[fp8_dequantize] {N}x{K}")
    w = synth.fp8_normal(8, "f8.deq", N, K, 0.02)
    out = torch.empty((N, K), dtype=torch.float32, device="cuda")
    binding.fp8_dequantize(dev_u8(w), out)
    ref = of8.decode_matrix(w, N, K).astype(np.float32)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("N,K", [(16, 256), (48, 768), (5120, 4096)])
def test_fp8_to_tiled_byte_exact(N, K):
    say(f"[fp8_to_tiled] {N}x{K}")
    w = synth.fp8_normal(7, "f8.tiled", N, K, 0.02)
    got = dev_tiled(w, N, K).cpu().numpy()
    assert np.array_equal(got, tiled_reference(w, N, K))


def gemm_check(w, x, N, K, M):
    wd = dev_tiled(w, N, K)
    y = torch.empty((M, N), dtype=torch.int16, device="cuda")
    ws = torch.empty(binding.fp8_gemm_tiled_workspace_bytes(M, N, K), dtype=torch.uint8,
                     device="cuda")
    binding.fp8_gemm_tiled(wd, dev_bf16(x), y, ws)
    # the row-major entry point regroups in its workspace and must give the same bits
    y2 = torch.empty_like(y)
    ws2 = torch.empty(binding.fp8_gemm_workspace_bytes(M, N, K), dtype=torch.uint8,
                      device="cuda")
    binding.fp8_gemm(dev_u8(w), dev_bf16(x), y2, ws2)
    assert torch.equal(y, y2)
    got = bf16_to_f64(y.cpu().numpy().view(np.uint16))
    ref = bf16_to_f64(x) @ of8.decode_matrix(w, N, K).T
    assert np.isfinite(got).all()
    err = np.abs(got - ref)
    # output rounded to bf16 (<= 2^-9 relative) plus fp32 accumulation
    bound = 2.0 ** -8 * np.abs(ref) + 1e-5 * np.sqrt(np.mean(ref ** 2))
    assert np.all(err <= bound), float((err / np.maximum(bound, 1e-30)).max())
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


@pytest.mark.parametrize("name,N,K", synth.GEMM_SHAPES)
def test_fp8_gemm_drafter_shapes_m8(name, N, K):
    say(f"[fp8_gemm] {name} M=8 {N}x{K}")
    w = synth.fp8_normal(synth.GEMM_SEED, f"gemm.{name}", N, K, 0.02)
    x = synth.normal_bf16(synth.GEMM_SEED, f"gemm.{name}.x", (8, K), 1.0)
    rel = gemm_check(w, x, N, K, 8)
    assert rel < 3e-3


@pytest.mark.parametrize("M,K", [(1, 2048), (3, 2048), (16, 2048), (1, 1280), (16, 1280),
                                 (17, 1280), (40, 2048), (128, 1280), (300, 2048)])
def test_fp8_gemm_row_counts(M, K):
    """Ragged row counts: up to 16 rows with K % 1024 == 0 the streaming kernel, the rest
    the many-row kernel (ragged row and column tiles)."""
    N = 272
    say(f"[fp8_gemm] M={M} {N}x{K}")
    w = synth.fp8_normal(5, "f8.rows", N, K, 0.02)
    x = synth.normal_bf16(5, "f8.rows.x", (M, K), 1.0)
    gemm_check(w, x, N, K, M)


@pytest.mark.parametrize("M,N,K", [(160, 4096, 4096), (256, 8704, 5120), (136, 34816, 4096)])
def test_fp8_gemm_schedules(M, N, K):
    """Many-row GEMM schedules: one round of K splits (16 and 34 tiles), stream-K (136)."""
    say(f"[fp8_gemm schedules] M={M} {N}x{K}")
    w = synth.fp8_normal(8, "f8.sk", N, K, 0.02)
    x = synth.normal_bf16(8, "f8.sk.x", (M, K), 1.0)
    gemm_check(w, x, N, K, M)


@pytest.mark.parametrize("M", [8, 16, 40])
def test_fp8_gemm_arbitrary_codes(M):
    """Codes the packer never writes (any finite code, subnormals included) and row
    scales of both signs over a wide range, through the streaming (8, 16 rows) and the
    many-row kernel (40)."""
    N, K = 64, 2048
    say(f"[fp8 arbitrary] GEMM M={M} {N}x{K}")
    rng = np.random.default_rng(30 + M)
    codes = rng.integers(0, 256, (N, K), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] ^= 0x01                      # no NaN codes
    scales = (rng.choice([-1.0, 1.0], N) * 2.0 ** rng.uniform(-20, 4, N)).astype(np.float32)
    w = make_matrix(codes, scales)
    x = (rng.standard_normal((M, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    gemm_check(w, x, N, K, M)


@pytest.mark.parametrize("shape,batch", [("mid", 1), ("mid", 2), ("mid", 16), ("tiny", 2)])
def test_small_step_fp8(shape, batch):
    """Whole draft steps with FP8 weights: a 2-layer drafter whose products all take the
    streaming kernel (1 sequence) or the many-row one (2 sequences: 32 MLP rows; 16
    sequences: 256 MLP rows over two row tiles), and the tiny drafter (K = 256 and 1280:
    the many-row kernel)."""
    s = dataclasses.replace(synth.MID if shape == "mid" else synth.TINY, weight_fmt="fp8")
    wl = dataclasses.replace(synth.WORKLOADS["tiny"], shape=s, batch=batch, ctx_len=96,
                             seed=60 + batch)
    say(f"[step fp8] {shape} batch {batch}")
    bufs = runner.StepBuffers(wl)
    bufs.step()
    torch.cuda.synchronize()
    ref = parity.run_oracle(wl, bufs.host_W, bufs.inputs)
    g = full_check(wl, bufs, ref)
    check_verify(bufs, g)


@pytest.mark.timeout(900)
def test_full_step_b1_fp8_parity():
    """The pages' draft shape with FP8 drafter weights, one sequence, 4096 cached rows."""
    wl = synth.WORKLOADS["full_b1_fp8"]
    say(f"[step] {wl.name}: generating inputs")
    bufs = runner.StepBuffers(wl)
    say("  running GPU step")
    bufs.step()
    torch.cuda.synchronize()
    say("  running oracle")
    ref = parity.run_oracle(wl, bufs.host_W, bufs.inputs)
    g = full_check(wl, bufs, ref)
    check_verify(bufs, g)
