"""ctypes binding of libdflash.so: argument marshalling only.

Every step of the draft path runs in the library's HIP kernels; this module
passes device pointers (torch tensors' data_ptr()), sizes and the current HIP
stream, and turns negative status codes into exceptions.  PyTorch supplies
device memory and streams.  There is no CPU fallback: if the library is missing
it is built, and if it cannot be loaded the call fails.
"""
import ctypes
import os
import re

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdflash.so")
MAX_LAYERS = 8
BLOCK = 8

W_Q4K, W_BF16, W_Q8_0, W_FP8 = 0, 1, 2, 3
WEIGHT_FMT = {"q4k": W_Q4K, "bf16": W_BF16, "q8_0": W_Q8_0, "fp8": W_FP8}
PROBE_NONE, PROBE_LM_HEAD, PROBE_FFN_GATE_UP = 0, 1, 2
LAYOUT_ROWMAJOR, LAYOUT_TILED = 0, 0x444C4954
NOALLOC_SCRATCH_BYTES = 32 << 20        # DFLASH_NOALLOC_SCRATCH_BYTES
STATUS = {0: "OK", -1: "EINVAL", -2: "ESHAPE", -3: "EALIGN", -4: "EWORKSPACE", -5: "EHIP",
          -6: "ELAYOUT", -7: "ESCRATCH"}

c_int, c_float, c_void_p, c_size_t = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t


class Config(ctypes.Structure):
    _fields_ = [(n, c_int) for n in ("n_layers", "hidden", "ffn", "n_q_heads", "n_kv_heads",
                                     "head_dim", "window", "vocab", "n_taps", "block", "top_k",
                                     "sel_rank", "weight_fmt")] + \
               [(n, c_float) for n in ("rms_eps", "rope_theta", "pair_scale")]


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("wq", "wk", "wv", "wo", "wg", "wu", "wd", "in_norm",
                                        "post_norm", "q_norm", "k_norm", "w_conv")]


class Weights(ctypes.Structure):
    _fields_ = [("fc", c_void_p), ("hidden_norm", c_void_p),
                ("layer", LayerWeights * MAX_LAYERS)] + \
               [(n, c_void_p) for n in ("final_norm", "embed", "lm_head", "mask_emb", "sel_proj",
                                        "code_a", "code_b")] + \
               [("linear_layout", ctypes.c_uint32)]


class Probe(ctypes.Structure):
    _fields_ = [("kernel", c_int), ("layer", c_int), ("ev_start", c_void_p), ("ev_stop", c_void_p)]


class DflashError(RuntimeError):
    pass


_lib = None


def lib():
    """Load libdflash.so (building it first if it is not there)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build
        build.build()
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    L.dflash_workspace_bytes.argtypes = [P(Config), c_int, c_int]
    L.dflash_workspace_bytes.restype = c_size_t
    L.dflash_draft_step.argtypes = [P(Config), P(Weights), c_int, c_void_p, c_int, c_void_p,
                                    c_void_p, c_void_p, c_void_p, c_int, c_void_p, c_void_p,
                                    c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, P(Probe),
                                    c_void_p]
    L.dflash_draft_step.restype = c_int
    L.dflash_draft_step_noalloc.argtypes = [P(Config), P(Weights), c_int, c_void_p, c_int,
                                            c_void_p, c_void_p, c_void_p, c_void_p, c_int,
                                            c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                            c_void_p]
    L.dflash_draft_step_noalloc.restype = c_int
    L.dflash_verify_prefix.argtypes = [c_void_p, c_void_p, c_int, c_int, c_void_p, c_void_p,
                                       c_void_p]
    L.dflash_verify_prefix.restype = c_int
    L.dflash_verify_sampled_workspace_bytes.argtypes = [c_int, c_int, c_int]
    L.dflash_verify_sampled_workspace_bytes.restype = c_size_t
    L.dflash_verify_sampled.argtypes = [c_void_p, c_void_p, c_void_p, c_int, c_int, c_int,
                                        c_float, c_int, c_float, c_void_p, c_size_t, c_void_p,
                                        c_void_p, c_void_p]
    L.dflash_verify_sampled.restype = c_int
    L.q4k_gemm_workspace_bytes.argtypes = [c_int, c_int, c_int]
    L.q4k_gemm_workspace_bytes.restype = c_size_t
    L.q4k_gemm.argtypes = [c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_void_p, c_size_t,
                           c_void_p]
    L.q4k_gemm.restype = c_int
    L.q4k_gemm_tiled_workspace_bytes.argtypes = [c_int, c_int, c_int]
    L.q4k_gemm_tiled_workspace_bytes.restype = c_size_t
    L.q4k_gemm_tiled.argtypes = [c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_void_p,
                                 c_size_t, c_void_p]
    L.q4k_gemm_tiled.restype = c_int
    L.q4k_dequantize.argtypes = [c_void_p, c_void_p, ctypes.c_longlong, c_void_p]
    L.q4k_dequantize.restype = c_int
    L.q4k_to_tiled.argtypes = [c_void_p, c_void_p, c_int, c_int, c_void_p]
    L.q4k_to_tiled.restype = c_int
    L.q8_0_gemm_workspace_bytes.argtypes = [c_int, c_int, c_int]
    L.q8_0_gemm_workspace_bytes.restype = c_size_t
    L.q8_0_gemm.argtypes = [c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_void_p,
                            c_size_t, c_void_p]
    L.q8_0_gemm.restype = c_int
    L.q8_0_gemm_tiled_workspace_bytes.argtypes = [c_int, c_int, c_int]
    L.q8_0_gemm_tiled_workspace_bytes.restype = c_size_t
    L.q8_0_gemm_tiled.argtypes = [c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_void_p,
                                  c_size_t, c_void_p]
    L.q8_0_gemm_tiled.restype = c_int
    L.q8_0_to_tiled.argtypes = [c_void_p, c_void_p, c_int, c_int, c_void_p]
    L.q8_0_to_tiled.restype = c_int
    L.q8_0_dequantize.argtypes = [c_void_p, c_void_p, ctypes.c_longlong, c_void_p]
    L.q8_0_dequantize.restype = c_int
    L.fp8_gemm_workspace_bytes.argtypes = [c_int, c_int, c_int]
    L.fp8_gemm_workspace_bytes.restype = c_size_t
    L.fp8_gemm.argtypes = [c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_void_p,
                           c_size_t, c_void_p]
    L.fp8_gemm.restype = c_int
    L.fp8_gemm_tiled_workspace_bytes.argtypes = [c_int, c_int, c_int]
    L.fp8_gemm_tiled_workspace_bytes.restype = c_size_t
    L.fp8_gemm_tiled.argtypes = [c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_void_p,
                                 c_size_t, c_void_p]
    L.fp8_gemm_tiled.restype = c_int
    L.fp8_to_tiled.argtypes = [c_void_p, c_void_p, c_int, c_int, c_void_p]
    L.fp8_to_tiled.restype = c_int
    L.fp8_dequantize.argtypes = [c_void_p, c_void_p, c_int, c_int, c_void_p]
    L.fp8_dequantize.restype = c_int
    L.dflash_status_str.argtypes = [c_int]
    L.dflash_status_str.restype = ctypes.c_char_p
    _lib = L
    return L


EXPORTS = ["dflash_workspace_bytes", "dflash_draft_step", "dflash_verify_prefix",
           "dflash_draft_step_noalloc",
           "dflash_verify_sampled_workspace_bytes", "dflash_verify_sampled",
           "q4k_gemm_workspace_bytes", "q4k_gemm", "q4k_gemm_tiled_workspace_bytes",
           "q4k_gemm_tiled", "q4k_to_tiled", "q4k_dequantize",
           "q8_0_gemm_workspace_bytes", "q8_0_gemm", "q8_0_gemm_tiled_workspace_bytes",
           "q8_0_gemm_tiled", "q8_0_to_tiled", "q8_0_dequantize",
           "fp8_gemm_workspace_bytes", "fp8_gemm", "fp8_gemm_tiled_workspace_bytes",
           "fp8_gemm_tiled", "fp8_to_tiled", "fp8_dequantize",
           "dflash_status_str"]


def check(rc):
    if rc != 0:
        raise DflashError(f"dflash status {rc} ({STATUS.get(rc, '?')}): "
                          f"{lib().dflash_status_str(rc).decode()}")


def make_config(shape):
    """Config struct from a synth.Shape-like object."""
    return Config(shape.n_layers, shape.hidden, shape.ffn, shape.n_q, shape.n_kv, shape.head_dim,
                  shape.window, shape.vocab, shape.n_taps, shape.block, shape.top_k,
                  shape.sel_rank, WEIGHT_FMT[shape.weight_fmt],
                  shape.rms_eps, shape.rope_theta, shape.pair_scale)


def workspace_bytes(cfg, batch, t_new):
    n = lib().dflash_workspace_bytes(ctypes.byref(cfg), batch, t_new)
    if n == 0:
        raise DflashError("unsupported configuration")
    return n


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _linear_dims(s):
    """(rows = out, cols = in) of each linear weight field of the weights struct."""
    qd, kd, H = s.n_q * s.head_dim, s.n_kv * s.head_dim, s.hidden
    dims = {"fc": (H, s.n_taps * H)}
    for l in range(s.n_layers):
        dims.update({f"l{l}.wq": (qd, H), f"l{l}.wk": (kd, H), f"l{l}.wv": (kd, H),
                     f"l{l}.wo": (H, qd), f"l{l}.wg": (s.ffn, H), f"l{l}.wu": (s.ffn, H),
                     f"l{l}.wd": (H, s.ffn)})
    return dims


class DeviceWeights:
    """Drafter weights resident in device memory, plus the C struct pointing at them.

    `W` is the host weight dict of synth.make_weights (linear weights as
    ("q4k" / "q8_0" / "fp8", row-major bytes) or ("bf16", uint16 array); the rest uint16
    arrays).  Q4_K, Q8_0 and FP8 matrices are regrouped on the device into the library's
    tiled layouts (q4k_to_tiled, q8_0_to_tiled, fp8_to_tiled) after the upload.
    """

    def __init__(self, shape, W, device="cuda"):
        import torch
        self.shape = shape
        self.tensors = {}
        shared = {}
        dims = _linear_dims(shape)

        def up(name, arr, fmt):
            arr = np.ascontiguousarray(arr)
            key = arr.__array_interface__["data"][0]
            if key in shared:                      # tied embedding / output head
                t = shared[key]
            else:
                dt = torch.uint8 if arr.dtype == np.uint8 else torch.int16
                t = torch.from_numpy(arr.view(np.uint8 if arr.dtype == np.uint8 else np.int16))
                t = t.to(device, dtype=dt)
                if fmt in ("q4k", "q8_0", "fp8"):
                    tiled = torch.empty_like(t)
                    {"q4k": q4k_to_tiled, "q8_0": q8_0_to_tiled,
                     "fp8": fp8_to_tiled}[fmt](t, tiled, *dims[name])
                    t = tiled
                shared[key] = t
            self.tensors[name] = t
            return t.data_ptr()

        s = Weights()
        s.linear_layout = LAYOUT_TILED          # quantised matrices are regrouped below
        for name, val in W.items():
            arr = val[1] if isinstance(val, tuple) else val
            p = up(name, arr, val[0] if isinstance(val, tuple) else "bf16")
            m = re.match(r"^l(\d+)\.(\w+)$", name)
            if m:
                setattr(s.layer[int(m.group(1))], m.group(2), p)
            else:
                setattr(s, name, p)
        self.struct = s


def draft_step(cfg, dw, taps, last_token, ctx_len, k_cache, v_cache, draft_tokens, cand_ids,
               cand_logp, workspace, dbg_hidden=None, dbg_logits=None, probe=None):
    """Enqueue one draft step on the current stream (all arguments torch tensors on device)."""
    B, t_new = taps.shape[0], taps.shape[1]
    cap = k_cache.shape[3]
    rc = lib().dflash_draft_step(ctypes.byref(cfg), ctypes.byref(dw.struct), B, _ptr(taps), t_new,
                                 _ptr(last_token), _ptr(ctx_len), _ptr(k_cache), _ptr(v_cache),
                                 cap, _ptr(draft_tokens), _ptr(cand_ids), _ptr(cand_logp),
                                 _ptr(dbg_hidden), _ptr(dbg_logits), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(),
                                 None if probe is None else ctypes.byref(probe), _stream())
    check(rc)


def draft_step_noalloc(cfg, dw, taps, last_token, ctx_len, k_cache, v_cache, draft_tokens,
                       cand_ids, cand_logp, dbg_hidden=None, dbg_logits=None):
    """Enqueue one draft step on the library's static device scratch (no workspace)."""
    B, t_new = taps.shape[0], taps.shape[1]
    cap = k_cache.shape[3]
    check(lib().dflash_draft_step_noalloc(ctypes.byref(cfg), ctypes.byref(dw.struct), B,
                                          _ptr(taps), t_new, _ptr(last_token), _ptr(ctx_len),
                                          _ptr(k_cache), _ptr(v_cache), cap, _ptr(draft_tokens),
                                          _ptr(cand_ids), _ptr(cand_logp), _ptr(dbg_hidden),
                                          _ptr(dbg_logits), _stream()))


def verify_prefix(draft, target, accept_len, out_tokens):
    B, n = draft.shape
    check(lib().dflash_verify_prefix(_ptr(draft), _ptr(target), B, n, _ptr(accept_len),
                                     _ptr(out_tokens), _stream()))


def verify_sampled_workspace_bytes(batch, n, vocab):
    return lib().dflash_verify_sampled_workspace_bytes(batch, n, vocab)


def verify_sampled(draft, target_logits, uniforms, temperature, top_k, top_p, workspace,
                   accept_len, out_tokens):
    """Enqueue sampled acceptance (device tensors: draft int32 [B, n], target_logits fp32
    [B, n + 1, V], uniforms fp32 [B, n + 1, 2], outputs int32 [B] and [B, n + 1])."""
    B, n = draft.shape
    V = target_logits.shape[2]
    check(lib().dflash_verify_sampled(_ptr(draft), _ptr(target_logits), _ptr(uniforms), B, n, V,
                                      temperature, top_k, top_p, _ptr(workspace),
                                      workspace.numel() * workspace.element_size(),
                                      _ptr(accept_len), _ptr(out_tokens), _stream()))


def q4k_gemm(w, x, y, workspace):
    M, K = x.shape
    N = y.shape[1]
    check(lib().q4k_gemm(_ptr(w), _ptr(x), _ptr(y), M, N, K, _ptr(workspace),
                         workspace.numel() * workspace.element_size(), _stream()))


def q4k_gemm_workspace_bytes(M, N, K):
    return lib().q4k_gemm_workspace_bytes(M, N, K)


def q4k_gemm_tiled(w, x, y, workspace):
    M, K = x.shape
    N = y.shape[1]
    check(lib().q4k_gemm_tiled(_ptr(w), _ptr(x), _ptr(y), M, N, K, _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream()))


def q4k_gemm_tiled_workspace_bytes(M, N, K):
    return lib().q4k_gemm_tiled_workspace_bytes(M, N, K)


def q4k_to_tiled(src, dst, N, K):
    """Regroup a row-major Q4_K matrix [N][K] (device uint8) into the tiled layout."""
    check(lib().q4k_to_tiled(_ptr(src), _ptr(dst), N, K, _stream()))


def q8_0_gemm(w, x, y, workspace):
    M, K = x.shape
    N = y.shape[1]
    check(lib().q8_0_gemm(_ptr(w), _ptr(x), _ptr(y), M, N, K, _ptr(workspace),
                          workspace.numel() * workspace.element_size(), _stream()))


def q8_0_gemm_workspace_bytes(M, N, K):
    return lib().q8_0_gemm_workspace_bytes(M, N, K)


def q8_0_gemm_tiled(w, x, y, workspace):
    M, K = x.shape
    N = y.shape[1]
    check(lib().q8_0_gemm_tiled(_ptr(w), _ptr(x), _ptr(y), M, N, K, _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream()))


def q8_0_gemm_tiled_workspace_bytes(M, N, K):
    return lib().q8_0_gemm_tiled_workspace_bytes(M, N, K)


def q8_0_to_tiled(src, dst, N, K):
    """Regroup a row-major Q8_0 matrix [N][K] (device uint8) into the tiled layout."""
    check(lib().q8_0_to_tiled(_ptr(src), _ptr(dst), N, K, _stream()))


def q8_0_dequantize(w, out):
    check(lib().q8_0_dequantize(_ptr(w), _ptr(out), out.numel() // 32, _stream()))


def fp8_gemm(w, x, y, workspace):
    M, K = x.shape
    N = y.shape[1]
    check(lib().fp8_gemm(_ptr(w), _ptr(x), _ptr(y), M, N, K, _ptr(workspace),
                         workspace.numel() * workspace.element_size(), _stream()))


def fp8_gemm_workspace_bytes(M, N, K):
    return lib().fp8_gemm_workspace_bytes(M, N, K)


def fp8_gemm_tiled(w, x, y, workspace):
    M, K = x.shape
    N = y.shape[1]
    check(lib().fp8_gemm_tiled(_ptr(w), _ptr(x), _ptr(y), M, N, K, _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream()))


def fp8_gemm_tiled_workspace_bytes(M, N, K):
    return lib().fp8_gemm_tiled_workspace_bytes(M, N, K)


def fp8_to_tiled(src, dst, N, K):
    """Regroup a row-major FP8 matrix [N][K] (+ row scales; device uint8) into the tiled layout."""
    check(lib().fp8_to_tiled(_ptr(src), _ptr(dst), N, K, _stream()))


def fp8_dequantize(w, out):
    """out: fp32 [N, K] device tensor; w: the matrix's N K + 4 N bytes."""
    N, K = out.shape
    check(lib().fp8_dequantize(_ptr(w), _ptr(out), N, K, _stream()))


def q4k_dequantize(w, out):
    check(lib().q4k_dequantize(_ptr(w), _ptr(out), out.numel() // 256, _stream()))


# ---------------------------------------------------------------------------
# HIP events for live per-kernel timing (recorded by the library on its stream)
# ---------------------------------------------------------------------------
_hip = None


def hip():
    global _hip
    if _hip is None:
        h = ctypes.CDLL("libamdhip64.so")
        h.hipEventCreate.argtypes = [ctypes.POINTER(c_void_p)]
        h.hipEventDestroy.argtypes = [c_void_p]
        h.hipEventSynchronize.argtypes = [c_void_p]
        h.hipEventElapsedTime.argtypes = [ctypes.POINTER(c_float), c_void_p, c_void_p]
        h.hipEventRecord.argtypes = [c_void_p, c_void_p]
        _hip = h
    return _hip


class HipEvent:
    def __init__(self):
        self.ev = c_void_p()
        rc = hip().hipEventCreate(ctypes.byref(self.ev))
        if rc != 0:
            raise DflashError(f"hipEventCreate failed: {rc}")

    def record(self):
        hip().hipEventRecord(self.ev, _stream())

    def elapsed_ms(self, later):
        hip().hipEventSynchronize(later.ev)
        ms = c_float()
        rc = hip().hipEventElapsedTime(ctypes.byref(ms), self.ev, later.ev)
        if rc != 0:
            raise DflashError(f"hipEventElapsedTime failed: {rc}")
        return ms.value

    def __del__(self):
        try:
            if self.ev:
                hip().hipEventDestroy(self.ev)
        except Exception:
            pass


def make_probe(kernel, start, stop, layer=0):
    return Probe(kernel, layer, start.ev, stop.ev)
