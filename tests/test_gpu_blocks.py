"""GPU decode and GEMMs on quantised blocks the host packer never makes (GPU).

The packer writes d, dmin >= 0 and scales from its own fit; the GPU kernels must
decode any block of the format.  The hand-made golden blocks (tests/golden/, their
values worked out by hand from the block layout) and blocks of arbitrary bytes with
finite fp16 scales (negative, subnormal and large ones included) go through
q4k_dequantize / q8_0_dequantize (bit-exact against the oracle) and through the
GEMM entry points (row-major and tiled; up to 16 rows the streaming kernels, above
the many-row kernel), whose outputs must match the oracle's float64 product to the
bf16 rounding of the output.  Q4_K: FastFlowLM card "Qwen3.8-27B-DFlash2-NPU2",
"Weights" row; Q8_0: Mindket kit page "Qwen3.8-27B-DFlash2-GGUF by z-lab",
draft-file table.
"""
import sys

import numpy as np
import pytest
import torch

from block_diffusion_draft_amd import binding
from oracle import q4k as oq4k
from oracle import q8_0 as oq8
from oracle.bf16 import bf16_to_f64
from tests.test_oracle_q4k import load_golden as q4k_golden
from tests.test_oracle_q8_0 import read_golden as q8_golden

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def finite_fp16(rng, n):
    """n fp16 bit patterns: finite, both signs, exponents across the normal range up to
    2^4 and about one in eight subnormal."""
    sign = rng.integers(0, 2, n).astype(np.uint16) << 15
    exp = rng.integers(1, 20, n).astype(np.uint16)          # 2^-14 .. 2^4
    exp[rng.random(n) < 0.125] = 0                            # subnormal
    man = rng.integers(0, 1024, n).astype(np.uint16)
    return sign | (exp << 10) | man


def random_q4k_blocks(seed, nblocks):
    rng = np.random.default_rng(seed)
    b = rng.integers(0, 256, (nblocks, 144), dtype=np.uint8)
    b[:, 0:2] = finite_fp16(rng, nblocks).view(np.uint8).reshape(nblocks, 2)
    b[:, 2:4] = finite_fp16(rng, nblocks).view(np.uint8).reshape(nblocks, 2)
    return b.reshape(-1)


def random_q8_blocks(seed, nblocks):
    rng = np.random.default_rng(seed)
    b = rng.integers(0, 256, (nblocks, 34), dtype=np.uint8)
    b[:, 0:2] = finite_fp16(rng, nblocks).view(np.uint8).reshape(nblocks, 2)
    return b.reshape(-1)


def q4k_matrix_with_golden(N, K, seed):
    """Random blocks with the hand-made block at the first super-block of every row."""
    w = random_q4k_blocks(seed, N * (K // 256)).reshape(N, K // 256, 144)
    w[:, 0] = q4k_golden()[0]
    return w.reshape(-1)


def q8_matrix_with_golden(N, K, seed):
    w = random_q8_blocks(seed, N * (K // 32)).reshape(N, K // 32, 34)
    w[:, 0] = q8_golden()[0]
    return w.reshape(-1)


def test_q4k_dequantize_golden_and_arbitrary_blocks():
    blk = q4k_golden()[0]
    w = np.concatenate([blk, random_q4k_blocks(1, 4095)])
    out = torch.empty(4096 * 256, dtype=torch.float32, device="cuda")
    binding.q4k_dequantize(dev(w), out)
    got = out.cpu().numpy()
    ref = oq4k.decode_blocks(w.reshape(-1, 144)).astype(np.float32).reshape(-1)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    # the hand-made block's values as worked out by hand
    _, d, dmin, sc, m = q4k_golden()
    for i in range(256):
        c, r = divmod(i, 64)
        q = (r & 15) if r < 32 else 2 * c + ((r - 32) >> 4)
        assert got[i] == d * sc[i // 32] * q - dmin * m[i // 32]


def test_q8_0_dequantize_golden_and_arbitrary_blocks():
    blk, want = q8_golden()
    w = np.concatenate([blk, random_q8_blocks(2, 4095)])
    out = torch.empty(4096 * 32, dtype=torch.float32, device="cuda")
    binding.q8_0_dequantize(dev(w), out)
    got = out.cpu().numpy()
    ref = oq8.decode_blocks(w.reshape(-1, 34)).astype(np.float32).reshape(-1)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert np.array_equal(got[:32], np.asarray(want, dtype=np.float32))


def check_product(fmt, w, N, K, M, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((M, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    xd = dev(x.view(np.int16))
    gemm, gemm_t = ((binding.q4k_gemm, binding.q4k_gemm_tiled) if fmt == "q4k" else
                    (binding.q8_0_gemm, binding.q8_0_gemm_tiled))
    wsb, wsb_t = ((binding.q4k_gemm_workspace_bytes, binding.q4k_gemm_tiled_workspace_bytes)
                  if fmt == "q4k" else
                  (binding.q8_0_gemm_workspace_bytes, binding.q8_0_gemm_tiled_workspace_bytes))
    to_tiled = binding.q4k_to_tiled if fmt == "q4k" else binding.q8_0_to_tiled
    wd = dev(w)
    y = torch.empty((M, N), dtype=torch.int16, device="cuda")
    gemm(wd, xd, y, torch.empty(wsb(M, N, K), dtype=torch.uint8, device="cuda"))
    wt = torch.empty_like(wd)
    to_tiled(wd, wt, N, K)
    y2 = torch.empty_like(y)
    gemm_t(wt, xd, y2, torch.empty(wsb_t(M, N, K), dtype=torch.uint8, device="cuda"))
    assert torch.equal(y, y2)
    got = bf16_to_f64(y.cpu().numpy().view(np.uint16))
    W = (oq4k.decode_matrix(w, N, K) if fmt == "q4k" else oq8.decode_matrix(w, N, K))
    ref = bf16_to_f64(x) @ W.T
    assert np.isfinite(got).all()
    bound = 2.0 ** -8 * np.abs(ref) + 1e-5 * np.sqrt(np.mean(ref ** 2))
    err = np.abs(got - ref)
    assert np.all(err <= bound), float((err / bound).max())


@pytest.mark.parametrize("M", [8, 16, 40])
def test_q4k_gemm_arbitrary_blocks(M):
    """Streaming kernel (8, 16 rows; K / 256 a multiple of 4) and many-row kernel (40)."""
    N, K = 64, 2048
    say(f"[q4k blocks] GEMM M={M} {N}x{K}")
    check_product("q4k", q4k_matrix_with_golden(N, K, 10 + M), N, K, M, 20 + M)


@pytest.mark.parametrize("M", [8, 16, 40])
def test_q8_0_gemm_arbitrary_blocks(M):
    N, K = 64, 2048
    say(f"[q8_0 blocks] GEMM M={M} {N}x{K}")
    check_product("q8_0", q8_matrix_with_golden(N, K, 30 + M), N, K, M, 40 + M)
