"""The C-ABI library: it loads, exports every declared entry point, and rejects bad
arguments on the host before touching a device (CPU only: no compute calls)."""
import ctypes
import os
import re

import pytest

from block_diffusion_draft_amd import binding, synth

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "dflash.h")
FAKE = 0x10000          # a non-null, 16-byte aligned address that is never dereferenced


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("dflash_draft_step", "dflash_verify_prefix", "dflash_verify_sampled",
              "dflash_verify_sampled_workspace_bytes", "q4k_gemm", "q4k_to_tiled",
              "q4k_dequantize", "dflash_workspace_bytes", "q4k_gemm_workspace_bytes",
              "q4k_gemm_tiled", "q4k_gemm_tiled_workspace_bytes",
              "q8_0_gemm", "q8_0_gemm_workspace_bytes", "q8_0_gemm_tiled",
              "q8_0_gemm_tiled_workspace_bytes", "q8_0_to_tiled", "q8_0_dequantize",
              "fp8_gemm", "fp8_gemm_workspace_bytes", "fp8_gemm_tiled",
              "fp8_gemm_tiled_workspace_bytes", "fp8_to_tiled", "fp8_dequantize",
              "dflash_status_str"):
        assert n in names
    assert sorted(binding.EXPORTS) == names


def test_library_exports_every_declared_symbol():
    L = binding.lib()
    for n in declared_functions():
        assert hasattr(L, n), n


def test_status_strings():
    L = binding.lib()
    for rc in (0, -1, -2, -3, -4, -5, -6, -7):
        assert L.dflash_status_str(rc)
        assert b"unknown" not in L.dflash_status_str(rc)
    assert b"unknown" in L.dflash_status_str(42)


def tiny_cfg(**kw):
    s = synth.TINY
    c = binding.make_config(s)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_workspace_query():
    L = binding.lib()
    assert L.dflash_workspace_bytes(ctypes.byref(tiny_cfg()), 1, 8) > 0
    assert L.dflash_workspace_bytes(ctypes.byref(tiny_cfg(head_dim=96)), 1, 8) == 0
    assert L.dflash_workspace_bytes(ctypes.byref(tiny_cfg()), 1, 9) == 0
    assert L.dflash_workspace_bytes(ctypes.byref(tiny_cfg()), 0, 8) == 0
    assert L.dflash_workspace_bytes(None, 1, 8) == 0
    full = binding.make_config(synth.FULL)
    assert L.dflash_workspace_bytes(ctypes.byref(full), 16, 8) > \
        L.dflash_workspace_bytes(ctypes.byref(full), 1, 8)


def fake_weights(cfg):
    w = binding.Weights()
    for f in ("fc", "hidden_norm", "final_norm", "embed", "lm_head", "mask_emb", "sel_proj",
              "code_a", "code_b"):
        setattr(w, f, FAKE)
    for l in range(cfg.n_layers):
        for f, _ in binding.LayerWeights._fields_:
            setattr(w.layer[l], f, FAKE)
    w.linear_layout = binding.LAYOUT_TILED
    return w


def call_step(cfg, w, batch=1, t_new=8, taps=FAKE, ws=FAKE, ws_bytes=1 << 40, cap=64):
    L = binding.lib()
    return L.dflash_draft_step(ctypes.byref(cfg), ctypes.byref(w) if w is not None else None,
                               batch, taps, t_new, FAKE, FAKE, FAKE, FAKE, cap, FAKE, FAKE, FAKE,
                               None, None, ws, ws_bytes, None, None)


def L_ok(cfg):
    return binding.lib().dflash_workspace_bytes(ctypes.byref(cfg), 1, 8) > 0


def test_draft_step_rejects_bad_arguments_before_launch():
    cfg = tiny_cfg()
    w = fake_weights(cfg)
    assert call_step(cfg, None) == -1                       # EINVAL: no weights
    assert call_step(cfg, w, taps=None) == -1
    assert call_step(cfg, w, batch=0) == -1
    assert call_step(cfg, w, t_new=0) == -1
    assert call_step(cfg, w, t_new=9) == -1
    assert call_step(cfg, w, cap=4) == -1                   # cache smaller than t_new
    assert call_step(tiny_cfg(head_dim=96), w) == -2        # ESHAPE
    assert call_step(tiny_cfg(top_k=17), w) == -2
    assert call_step(tiny_cfg(block=9), w) == -2             # blocks of 2..8
    assert call_step(tiny_cfg(block=1), w) == -2
    assert call_step(tiny_cfg(n_q_heads=128, n_kv_heads=32, head_dim=64), w) == -2   # n_q <= 64
    assert call_step(tiny_cfg(n_kv_heads=3), w) == -2
    assert call_step(tiny_cfg(hidden=200), w) == -2
    assert call_step(tiny_cfg(sel_rank=48), w) == -2
    assert call_step(tiny_cfg(weight_fmt=7), w) == -1
    assert L_ok(tiny_cfg(weight_fmt=2))                      # Q8_0 is a supported format
    assert L_ok(tiny_cfg(weight_fmt=3))                      # and FP8
    assert call_step(tiny_cfg(weight_fmt=4), w) == -1
    assert call_step(cfg, w, taps=FAKE + 2) == -3           # EALIGN
    assert call_step(cfg, w, ws=None) == -4                 # EWORKSPACE
    assert call_step(cfg, w, ws_bytes=16) == -4
    assert call_step(cfg, w, ws=FAKE + 16) == -4            # workspace must be 256-aligned
    w.layer[0].wq = None
    assert call_step(cfg, w) == -1


def test_noalloc_step_checks_arguments_and_scratch_size_before_launch():
    """The no-allocation step validates like the workspace step, and refuses (before any
    HIP call) a configuration whose workspace exceeds its static scratch."""
    L = binding.lib()
    full = binding.make_config(synth.FULL)
    w = fake_weights(full)
    call = lambda cfg, b: L.dflash_draft_step_noalloc(ctypes.byref(cfg), ctypes.byref(w), b,
                                                      FAKE, 8, FAKE, FAKE, FAKE, FAKE, 64, FAKE,
                                                      FAKE, FAKE, None, None, None)
    assert binding.workspace_bytes(full, 16, 8) > binding.NOALLOC_SCRATCH_BYTES
    assert call(full, 16) == -7                             # ESCRATCH
    assert call(full, 0) == -1
    assert call(tiny_cfg(head_dim=96), 1) == -2
    w.linear_layout = 0
    assert call(full, 1) == -6


def test_draft_step_requires_the_tiled_layout_tag():
    """Quantised matrices are read in the tiled layout only; a weights struct that does
    not declare it (a zero-initialised tag says row-major) is refused before launch."""
    for fmt in (binding.W_Q4K, binding.W_Q8_0, binding.W_FP8):
        cfg = tiny_cfg(weight_fmt=fmt)
        w = fake_weights(cfg)
        w.linear_layout = binding.LAYOUT_ROWMAJOR
        assert call_step(cfg, w) == -6                      # ELAYOUT
        w.linear_layout = 0x12345678
        assert call_step(cfg, w) == -6
    cfg = tiny_cfg(weight_fmt=binding.W_BF16)                # bf16: row-major, tag ignored
    w = fake_weights(cfg)
    w.linear_layout = binding.LAYOUT_ROWMAJOR
    assert call_step(cfg, w, ws=None) == -4                  # passes the tag, stops at EWORKSPACE


def test_q4k_gemm_and_verify_reject_bad_arguments():
    L = binding.lib()
    assert L.q4k_gemm(FAKE, FAKE, FAKE, 8, 5120, 5000, FAKE, 1 << 40, None) == -2
    assert L.q4k_gemm(FAKE, FAKE, FAKE, 8, 5121, 5120, FAKE, 1 << 40, None) == -2
    assert L.q4k_gemm(FAKE, FAKE, FAKE, 0, 5120, 5120, FAKE, 1 << 40, None) == -2
    assert L.q4k_gemm(FAKE + 4, FAKE, FAKE, 8, 5120, 5120, FAKE, 1 << 40, None) == -3
    assert L.q4k_gemm(FAKE, FAKE, FAKE, 8, 5120, 5120, FAKE, 16, None) == -4
    assert L.q4k_gemm(None, FAKE, FAKE, 8, 5120, 5120, FAKE, 1 << 40, None) == -1
    assert L.q4k_gemm_workspace_bytes(8, 5120, 25600) > 0
    assert L.q4k_gemm_workspace_bytes(8, 5120, 100) == 0
    # row-major W: the workspace also holds the tiled copy of W
    assert L.q4k_gemm_workspace_bytes(8, 5120, 25600) >= \
        L.q4k_gemm_tiled_workspace_bytes(8, 5120, 25600) + 5120 * 100 * 144
    assert L.q4k_gemm_tiled(FAKE, FAKE, FAKE, 8, 5120, 5000, FAKE, 1 << 40, None) == -2
    assert L.q4k_gemm_tiled(FAKE + 4, FAKE, FAKE, 8, 5120, 5120, FAKE, 1 << 40, None) == -3
    assert L.q4k_gemm_tiled(FAKE, FAKE, FAKE, 8, 5120, 5120, FAKE, 16, None) == -4
    assert L.q4k_gemm_tiled(None, FAKE, FAKE, 8, 5120, 5120, FAKE, 1 << 40, None) == -1
    assert L.q4k_gemm(FAKE, FAKE, FAKE, 8, 5120, 5120, FAKE + 16, 1 << 40, None) == -4  # 256-aligned
    assert L.q4k_gemm(FAKE, FAKE, FAKE, 8, 5120, 5120, FAKE, 1 << 40, None) == -1  # W in workspace
    assert L.dflash_verify_prefix(FAKE, FAKE, 1, 0, FAKE, FAKE, None) == -1
    assert L.dflash_verify_prefix(None, FAKE, 1, 7, FAKE, FAKE, None) == -1
    assert L.q4k_dequantize(FAKE, FAKE, 0, None) == -1
    assert L.q4k_to_tiled(None, FAKE, 16, 256, None) == -1
    assert L.q4k_to_tiled(FAKE, FAKE + (1 << 30), 24, 256, None) == -2
    assert L.q4k_to_tiled(FAKE, FAKE + (1 << 30), 16, 300, None) == -2
    assert L.q4k_to_tiled(FAKE + 8, FAKE + (1 << 30), 16, 256, None) == -3
    assert L.q4k_to_tiled(FAKE, FAKE + 1024, 16, 256, None) == -1   # overlapping buffers


def test_q8_0_entries_reject_bad_arguments():
    L = binding.lib()
    assert L.q8_0_gemm(FAKE, FAKE, FAKE, 8, 5120, 5000, FAKE, 1 << 40, None) == -2
    assert L.q8_0_gemm(FAKE, FAKE, FAKE, 8, 5121, 5120, FAKE, 1 << 40, None) == -2
    assert L.q8_0_gemm(FAKE, FAKE, FAKE, 0, 5120, 5120, FAKE, 1 << 40, None) == -2
    assert L.q8_0_gemm(FAKE, FAKE, FAKE, 4097, 5120, 5120, FAKE, 1 << 40, None) == -2
    assert L.q8_0_gemm(FAKE + 4, FAKE, FAKE, 8, 5120, 5120, FAKE, 1 << 40, None) == -3
    assert L.q8_0_gemm(FAKE, FAKE, FAKE, 8, 5120, 5120, FAKE, 16, None) == -4
    assert L.q8_0_gemm(None, FAKE, FAKE, 8, 5120, 5120, FAKE, 1 << 40, None) == -1
    assert L.q8_0_gemm_workspace_bytes(8, 5120, 25600) > 0
    assert L.q8_0_gemm_workspace_bytes(300, 5120, 1280) >= 300 * 5120 * 4   # many-row GEMM
    assert L.q8_0_gemm_workspace_bytes(8, 5120, 100) == 0
    assert L.q8_0_gemm_tiled_workspace_bytes(300, 5120, 1280) >= 300 * 5120 * 4
    assert L.q8_0_gemm_workspace_bytes(8, 5120, 25600) >= \
        L.q8_0_gemm_tiled_workspace_bytes(8, 5120, 25600) + 5120 * 800 * 34
    assert L.q8_0_gemm_tiled(FAKE, FAKE, FAKE, 8, 5121, 5120, FAKE, 1 << 40, None) == -2
    assert L.q8_0_gemm_tiled(FAKE, FAKE, FAKE, 8, 5120, 5120, FAKE, 16, None) == -4
    assert L.q8_0_dequantize(FAKE, FAKE, 0, None) == -1
    assert L.q8_0_dequantize(FAKE + 2, FAKE, 1, None) == -3
    assert L.q8_0_to_tiled(None, FAKE, 16, 256, None) == -1
    assert L.q8_0_to_tiled(FAKE, FAKE + (1 << 30), 24, 256, None) == -2
    assert L.q8_0_to_tiled(FAKE, FAKE + (1 << 30), 16, 288, None) == -2
    assert L.q8_0_to_tiled(FAKE + 8, FAKE + (1 << 30), 16, 256, None) == -3
    assert L.q8_0_to_tiled(FAKE, FAKE + 1024, 16, 256, None) == -1   # overlapping buffers


def test_fp8_entries_reject_bad_arguments():
    L = binding.lib()
    assert L.fp8_gemm(FAKE, FAKE, FAKE, 8, 5120, 5000, FAKE, 1 << 40, None) == -2
    assert L.fp8_gemm(FAKE, FAKE, FAKE, 8, 5121, 5120, FAKE, 1 << 40, None) == -2
    assert L.fp8_gemm(FAKE, FAKE, FAKE, 0, 5120, 5120, FAKE, 1 << 40, None) == -2
    assert L.fp8_gemm(FAKE, FAKE, FAKE, 4097, 5120, 5120, FAKE, 1 << 40, None) == -2
    assert L.fp8_gemm(FAKE + 4, FAKE, FAKE, 8, 5120, 5120, FAKE, 1 << 40, None) == -3
    assert L.fp8_gemm(FAKE, FAKE, FAKE, 8, 5120, 5120, FAKE, 16, None) == -4
    assert L.fp8_gemm(None, FAKE, FAKE, 8, 5120, 5120, FAKE, 1 << 40, None) == -1
    assert L.fp8_gemm(FAKE, FAKE, FAKE, 8, 5120, 5120, FAKE, 1 << 40, None) == -1  # W in workspace
    # the row-major call holds the tiled copy (codes and row scales) before the partials
    assert L.fp8_gemm_workspace_bytes(8, 5120, 25600) >= \
        L.fp8_gemm_tiled_workspace_bytes(8, 5120, 25600) + 5120 * 25600 + 5120 * 4
    assert L.fp8_gemm_workspace_bytes(300, 5120, 1280) >= 300 * 5120 * 4     # many-row GEMM
    assert L.fp8_gemm_workspace_bytes(8, 5120, 100) == 0
    assert L.fp8_gemm_tiled(FAKE, FAKE, FAKE, 8, 5121, 5120, FAKE, 1 << 40, None) == -2
    assert L.fp8_gemm_tiled(FAKE, FAKE, FAKE, 8, 5120, 5120, FAKE, 16, None) == -4
    assert L.fp8_dequantize(None, FAKE, 4, 256, None) == -1
    assert L.fp8_dequantize(FAKE, FAKE, 0, 256, None) == -2
    assert L.fp8_dequantize(FAKE, FAKE, 4, 250, None) == -2
    assert L.fp8_dequantize(FAKE + 2, FAKE, 4, 256, None) == -3
    assert L.fp8_to_tiled(None, FAKE, 16, 256, None) == -1
    assert L.fp8_to_tiled(FAKE, FAKE + (1 << 30), 24, 256, None) == -2
    assert L.fp8_to_tiled(FAKE, FAKE + (1 << 30), 16, 288, None) == -2
    assert L.fp8_to_tiled(FAKE + 8, FAKE + (1 << 30), 16, 256, None) == -3
    assert L.fp8_to_tiled(FAKE, FAKE + 4096, 16, 256, None) == -1   # overlapping (4160 bytes)


def call_sampled(draft=FAKE, logits=FAKE, u=FAKE, batch=2, n=7, vocab=4096, T=1.0, k=20, p=0.95,
                 ws=FAKE, ws_bytes=1 << 40, acc=FAKE, out=FAKE):
    return binding.lib().dflash_verify_sampled(draft, logits, u, batch, n, vocab, T, k, p, ws,
                                               ws_bytes, acc, out, None)


def test_verify_sampled_rejects_bad_arguments_before_launch():
    L = binding.lib()
    assert L.dflash_verify_sampled_workspace_bytes(2, 7, 4096) > 0
    assert L.dflash_verify_sampled_workspace_bytes(2, 7, 248320) > \
        L.dflash_verify_sampled_workspace_bytes(1, 7, 248320)
    for bad in ((0, 7, 4096), (1, 0, 4096), (1, 64, 4096), (1, 7, 0), (1, 7, (1 << 20) + 1),
                (8192, 7, 4096)):
        assert L.dflash_verify_sampled_workspace_bytes(*bad) == 0, bad
    assert call_sampled(draft=None) == -1                   # EINVAL
    assert call_sampled(logits=None) == -1
    assert call_sampled(u=None) == -1
    assert call_sampled(out=None) == -1
    assert call_sampled(batch=0) == -1
    assert call_sampled(n=0) == -1
    assert call_sampled(T=0.0) == -1
    assert call_sampled(T=-1.0) == -1
    assert call_sampled(T=float("inf")) == -1
    assert call_sampled(T=float("nan")) == -1
    assert call_sampled(p=0.0) == -1
    assert call_sampled(p=1.01) == -1
    assert call_sampled(p=float("nan")) == -1
    assert call_sampled(k=0) == -1
    assert call_sampled(k=51, vocab=50) == -1               # top_k above the vocabulary
    assert call_sampled(n=64) == -2                         # ESHAPE
    assert call_sampled(k=65) == -2
    assert call_sampled(vocab=(1 << 20) + 1) == -2
    assert call_sampled(batch=8192) == -2                   # batch (n + 1) rows > 65535
    assert call_sampled(logits=FAKE + 2) == -3              # EALIGN
    assert call_sampled(acc=FAKE + 1) == -3
    assert call_sampled(ws=None) == -4                      # EWORKSPACE
    assert call_sampled(ws_bytes=16) == -4
    assert call_sampled(ws=FAKE + 4) == -4


def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return True


@pytest.mark.skipif(_gpu_visible(), reason="a GPU is visible: valid fake pointers would be used")
def test_valid_calls_without_a_gpu_return_ehip():
    """On a host without a GPU a call that passes every host check reaches its first
    HIP call, which fails: the status is DFLASH_EHIP, nothing crashes."""
    L = binding.lib()
    cfg = tiny_cfg()
    assert call_step(cfg, fake_weights(cfg), ws=FAKE * 256) == -5
    assert L.dflash_verify_prefix(FAKE, FAKE, 1, 7, FAKE, FAKE, None) == -5
    assert L.q4k_gemm_tiled(FAKE, FAKE, FAKE, 8, 5120, 5120, FAKE, 1 << 40, None) == -5
    assert L.q4k_dequantize(FAKE, FAKE, 1, None) == -5
