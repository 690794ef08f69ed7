"""Seeded synthetic inputs for the draft step, and a host-side Q4_K packer.

This module generates data and nothing else: it holds no step of the draft
forward.  The same arrays feed the GPU library and the reference checker.

Recipe (shapes and distributions follow the workloads the pages describe; the
pages measure on prompts and benchmark suites that are not available here, and
for the draft step only the shapes, the context length and the number of
appended rows matter, so seeded synthetic tensors stand in for them):
  * linear weights (fc, q/k/v/o, gate/up/down): N(0, 0.02), packed to Q4_K
    (or Q8_0, or FP8 E4M3 with a scale per row, or kept bf16 for the unquantised
    workload);
  * shared embedding / output head, dynamic-conv W_c, selector projection and
    codebooks, mask embedding: bf16 N(0, 0.02);
  * norm gains: 1.0 (``gain_jitter`` > 0 gives 1 + jitter * N(0, 1));
  * tapped target features: bf16 N(0, 1);
  * KV cache rows: bf16 N(0, 1) (only the rows a step can read are generated
    on the host; see ``WindowCache``);
  * last accepted tokens: uniform over the vocabulary.
Every tensor has its own stream of a counter-based generator keyed by
(seed, tensor name), so any slice can be regenerated exactly.
"""
import ctypes
import dataclasses
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csrc", "synth.c")
_LIB_PATH = os.path.join(_HERE, "libdflash_synth.so")
_lib = None


def build_synth(force=False):
    """Compile the generator/packer with gcc (-O3 -fopenmp) in-tree."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build_synth()
        L = ctypes.CDLL(_LIB_PATH)
        u64, i64, i32, f32, vp = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32,
                                  ctypes.c_float, ctypes.c_void_p)
        L.synth_normal_f32.argtypes = [u64, u64, u64, i64, f32, vp]
        L.synth_normal_bf16.argtypes = [u64, u64, u64, i64, f32, vp]
        L.synth_randint.argtypes = [u64, u64, i64, i32, i32, vp]
        L.synth_q4k_pack.argtypes = [vp, i64, i64, vp]
        L.synth_q4k_normal.argtypes = [u64, u64, i64, i64, f32, vp]
        L.synth_q8_0_pack.argtypes = [vp, i64, i64, vp]
        L.synth_q8_0_normal.argtypes = [u64, u64, i64, i64, f32, vp]
        L.synth_fp8_pack.argtypes = [vp, i64, i64, vp]
        L.synth_fp8_normal.argtypes = [u64, u64, i64, i64, f32, vp]
        for f in (L.synth_normal_f32, L.synth_normal_bf16, L.synth_randint,
                  L.synth_q4k_pack, L.synth_q4k_normal, L.synth_q8_0_pack,
                  L.synth_q8_0_normal, L.synth_fp8_pack, L.synth_fp8_normal):
            f.restype = None
        _lib = L
    return _lib


def stream_id(name):
    """FNV-1a 64-bit hash of a tensor name: the generator stream of that tensor."""
    h = 0xCBF29CE484222325
    for ch in name.encode():
        h ^= ch
        h = (h * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h


def normal_bf16(seed, name, shape, std=1.0, offset=0):
    out = np.empty(shape, dtype=np.uint16)
    lib().synth_normal_bf16(seed, stream_id(name), offset, out.size, std,
                            out.ctypes.data)
    return out


def normal_f32(seed, name, shape, std=1.0, offset=0):
    out = np.empty(shape, dtype=np.float32)
    lib().synth_normal_f32(seed, stream_id(name), offset, out.size, std, out.ctypes.data)
    return out


def randint(seed, name, shape, lo, hi):
    out = np.empty(shape, dtype=np.int32)
    lib().synth_randint(seed, stream_id(name), out.size, lo, hi, out.ctypes.data)
    return out


def uniform(seed, name, shape):
    """float32 uniform on [0, 1): multiples of 2^-24 (exact in float32 and float64)."""
    return randint(seed, name, shape, 0, 1 << 24).astype(np.float32) * np.float32(2.0 ** -24)


def target_logits(seed, name, draft, V, std=2.0, lift=0.9):
    """Synthetic target logits [B, n + 1, V] fp32 for drafted tokens draft [B, n]: N(0, std)
    per entry; at each proposal position, with probability `lift` (seeded), the drafted
    token's logit is set to the row maximum plus U(2, 7), so that the target usually
    ranks the draft first with a probability spread over roughly 0.4 .. 0.99, and the
    accepted lengths spread over 0 .. n."""
    draft = np.asarray(draft)
    B, n = draft.shape
    z = normal_f32(seed, name, (B, n + 1, V), std)
    coin = uniform(seed, name + ".lift", (B, n))
    off = uniform(seed, name + ".off", (B, n)) * np.float32(5.0) + np.float32(2.0)
    for b in range(B):
        for j in range(n):
            x = int(draft[b, j])
            if coin[b, j] < lift and 0 <= x < V:
                z[b, j, x] = z[b, j].max() + off[b, j]
    return z


def q4k_pack(w):
    """float32 [rows, cols] (cols % 256 == 0) -> Q4_K bytes uint8 [rows * cols/256 * 144]."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, cols = w.shape
    assert cols % 256 == 0
    out = np.empty(rows * (cols // 256) * 144, dtype=np.uint8)
    lib().synth_q4k_pack(w.ctypes.data, rows, cols, out.ctypes.data)
    return out


def q4k_normal(seed, name, rows, cols, std=0.02):
    """Q4_K bytes of a [rows, cols] matrix of std * N(0, 1) weights (stream `name`)."""
    assert cols % 256 == 0
    out = np.empty(rows * (cols // 256) * 144, dtype=np.uint8)
    lib().synth_q4k_normal(seed, stream_id(name), rows, cols, std, out.ctypes.data)
    return out


def q8_0_pack(w):
    """float32 [rows, cols] (cols % 32 == 0) -> Q8_0 bytes uint8 [rows * cols/32 * 34]."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, cols = w.shape
    assert cols % 32 == 0
    out = np.empty(rows * (cols // 32) * 34, dtype=np.uint8)
    lib().synth_q8_0_pack(w.ctypes.data, rows, cols, out.ctypes.data)
    return out


def q8_0_normal(seed, name, rows, cols, std=0.02):
    """Q8_0 bytes of a [rows, cols] matrix of std * N(0, 1) weights (stream `name`)."""
    assert cols % 32 == 0
    out = np.empty(rows * (cols // 32) * 34, dtype=np.uint8)
    lib().synth_q8_0_normal(seed, stream_id(name), rows, cols, std, out.ctypes.data)
    return out


def fp8_bytes(rows, cols):
    """Bytes of an FP8 matrix: one E4M3 code per weight, then one float32 scale per row."""
    return rows * cols + 4 * rows


def fp8_pack(w):
    """float32 [rows, cols] -> FP8 bytes uint8 [rows * cols + 4 rows] (codes, then scales)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, cols = w.shape
    assert cols % 2 == 0
    out = np.empty(fp8_bytes(rows, cols), dtype=np.uint8)
    lib().synth_fp8_pack(w.ctypes.data, rows, cols, out.ctypes.data)
    return out


def fp8_normal(seed, name, rows, cols, std=0.02):
    """FP8 bytes of a [rows, cols] matrix of std * N(0, 1) weights (stream `name`)."""
    assert cols % 2 == 0
    out = np.empty(fp8_bytes(rows, cols), dtype=np.uint8)
    lib().synth_fp8_normal(seed, stream_id(name), rows, cols, std, out.ctypes.data)
    return out


def bf16_from_f32(x):
    """float32 -> bf16 bits, round to nearest even (finite values)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


# ---------------------------------------------------------------------------
# shapes and workloads
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Shape:
    n_layers: int
    hidden: int
    ffn: int
    n_q: int
    n_kv: int
    head_dim: int
    window: int
    vocab: int
    top_k: int
    sel_rank: int
    n_taps: int = 5
    block: int = 8
    rms_eps: float = 1e-6
    rope_theta: float = 1e6
    weight_fmt: str = "q4k"

    @property
    def pair_scale(self):
        return 1.0 / float(np.sqrt(self.sel_rank))

    def as_dict(self):
        d = dataclasses.asdict(self)
        d["pair_scale"] = self.pair_scale
        return d


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    shape: Shape
    batch: int
    ctx_len: int          # rows cached before the step
    t_new: int            # context rows appended by the step
    seed: int
    cache_extra: int = 0  # spare rows beyond ctx_len + t_new

    @property
    def cache_cap(self):
        return self.ctx_len + self.t_new + self.cache_extra


TINY = Shape(n_layers=1, hidden=256, ffn=768, n_q=4, n_kv=2, head_dim=64, window=32,
             vocab=4096, top_k=4, sel_rank=32)
FULL = Shape(n_layers=5, hidden=5120, ffn=17408, n_q=32, n_kv=8, head_dim=128, window=2048,
             vocab=248320, top_k=16, sel_rank=256)
FULL_BF16 = dataclasses.replace(FULL, weight_fmt="bf16")
FULL_Q8_0 = dataclasses.replace(FULL, weight_fmt="q8_0")
FULL_FP8 = dataclasses.replace(FULL, weight_fmt="fp8")
# a mid-size drafter whose every product has K a multiple of 1024 (the 16-row Q8_0
# streaming kernel's split), small enough for the oracle in seconds
MID = Shape(n_layers=2, hidden=1024, ffn=2048, n_q=8, n_kv=2, head_dim=128, window=64,
            vocab=8192, top_k=16, sel_rank=64)

WORKLOADS = {
    "tiny": Workload("tiny-1L-h256-v4096-ctx48", TINY, batch=1, ctx_len=48, t_new=8, seed=0),
    "full_b1": Workload("dflash2-27b-draft-q4k-b1-ctx4096", FULL, batch=1, ctx_len=4096,
                        t_new=8, seed=3),
    "full_b16": Workload("dflash2-27b-draft-q4k-b16-ctx32768", FULL, batch=16,
                         ctx_len=32768, t_new=8, seed=4),
    "full_b64_bf16": Workload("dflash2-27b-draft-bf16-b64-ctx8192", FULL_BF16, batch=64,
                              ctx_len=8192, t_new=8, seed=5),
    "full_b1_q8_0": Workload("dflash2-27b-draft-q8_0-b1-ctx4096", FULL_Q8_0, batch=1,
                             ctx_len=4096, t_new=8, seed=6),
    "full_b1_fp8": Workload("dflash2-27b-draft-fp8-b1-ctx4096", FULL_FP8, batch=1,
                            ctx_len=4096, t_new=8, seed=7),
}

# the drafter's matrix shapes (name, N out, K in) at M = 8 activation rows
GEMM_SHAPES = [("fc", 5120, 25600), ("q", 4096, 5120), ("k", 1024, 5120), ("v", 1024, 5120),
               ("o", 5120, 4096), ("gate", 17408, 5120), ("up", 17408, 5120),
               ("down", 5120, 17408)]
GEMM_SEED = 1


def linear_shapes(s):
    """(name, rows=out, cols=in) of every linear weight of a drafter shape."""
    qd, kd = s.n_q * s.head_dim, s.n_kv * s.head_dim
    out = [("fc", s.hidden, s.n_taps * s.hidden)]
    for l in range(s.n_layers):
        out += [(f"l{l}.wq", qd, s.hidden), (f"l{l}.wk", kd, s.hidden),
                (f"l{l}.wv", kd, s.hidden), (f"l{l}.wo", s.hidden, qd),
                (f"l{l}.wg", s.ffn, s.hidden), (f"l{l}.wu", s.ffn, s.hidden),
                (f"l{l}.wd", s.hidden, s.ffn)]
    return out


def make_weights(s, seed, gain_jitter=0.0, code_std=0.02):
    """All drafter weights of shape `s` as a dict (the checker's format).

    Linear weights: ("q4k", "q8_0" or "fp8", uint8 bytes) or ("bf16", uint16 [rows, cols]).
    Everything else: uint16 bf16 arrays.  embed and lm_head are the same array
    (the draft shares the target's embedding table and output head).  code_std is
    the standard deviation of the two selector codebooks (``selector_codebooks``).
    """
    W = {}
    for name, rows, cols in linear_shapes(s):
        if s.weight_fmt == "q4k":
            W[name] = ("q4k", q4k_normal(seed, name, rows, cols, 0.02))
        elif s.weight_fmt == "q8_0":
            W[name] = ("q8_0", q8_0_normal(seed, name, rows, cols, 0.02))
        elif s.weight_fmt == "fp8":
            W[name] = ("fp8", fp8_normal(seed, name, rows, cols, 0.02))
        else:
            W[name] = ("bf16", normal_bf16(seed, name, (rows, cols), 0.02))

    def gain(name, n):
        if gain_jitter == 0.0:
            return np.full(n, 0x3F80, dtype=np.uint16)        # bf16 1.0
        return bf16_from_f32(1.0 + normal_f32(seed, name, (n,), gain_jitter))

    W["hidden_norm"] = gain("hidden_norm", s.hidden)
    W["final_norm"] = gain("final_norm", s.hidden)
    for l in range(s.n_layers):
        W[f"l{l}.in_norm"] = gain(f"l{l}.in_norm", s.hidden)
        W[f"l{l}.post_norm"] = gain(f"l{l}.post_norm", s.hidden)
        W[f"l{l}.q_norm"] = gain(f"l{l}.q_norm", s.head_dim)
        W[f"l{l}.k_norm"] = gain(f"l{l}.k_norm", s.head_dim)
        W[f"l{l}.w_conv"] = normal_bf16(seed, f"l{l}.w_conv",
                                        (2 * s.n_q, s.n_q * s.head_dim), 0.02)
    E = normal_bf16(seed, "embed", (s.vocab, s.hidden), 0.02)
    W["embed"] = E
    W["lm_head"] = E
    W["mask_emb"] = normal_bf16(seed, "mask_emb", (s.hidden,), 0.02)
    W["sel_proj"] = normal_bf16(seed, "sel_proj", (s.sel_rank, s.hidden), 0.02)
    W["code_a"], W["code_b"] = selector_codebooks(s, seed, code_std)
    return W


def selector_codebooks(s, seed, std=0.02):
    """The two [vocab, rank] bf16 selector codebooks, N(0, std).  At the workloads'
    std 0.02 the pair term s <A[u], B[v]> is about 4e-4, far below the gaps between
    candidate log-probabilities; std 1 makes it N(0, 1), so the transitions decide
    the selected path."""
    return (normal_bf16(seed, "code_a", (s.vocab, s.sel_rank), std),
            normal_bf16(seed, "code_b", (s.vocab, s.sel_rank), std))


class WindowCache:
    """The readable rows of a [L, B, n_kv, cap, d] bf16 cache, held on the host.

    Only rows [lo_b, ctx_len_b) per sequence are stored (lo_b = start of the
    attention window after the step appends t_new rows); indexing
    ``c[l, b, :, r0:r1, :]`` returns those rows and refuses anything else.
    """

    def __init__(self, rows, lo, shape):
        self.rows = rows            # list over b of uint16 [L, n_kv, S_b, d]
        self.lo = lo                # list over b
        self.shape = shape

    def __getitem__(self, idx):
        l, b, hs, rs, ds = idx
        r0, r1 = rs.start, rs.stop
        lo = self.lo[b]
        if r1 <= r0:
            return self.rows[b][l][hs, 0:0, ds]
        S = self.rows[b].shape[2]
        assert lo <= r0 and r1 <= lo + S, (r0, r1, lo, S)
        return self.rows[b][l][hs, r0 - lo:r1 - lo, ds]


def make_step_inputs(wl, ctx_len=None, full_cache=None):
    """Per-sequence inputs of one draft step of workload `wl`.

    Returns dict(taps [B, t_new, n_taps H] u16, last_token [B] i32, ctx_len [B] i32,
    k_cache, v_cache).  The caches are full uint16 arrays [L, B, n_kv, cap, d]
    when `full_cache` (default: when they are under 64 MiB), else WindowCache
    objects holding only the rows the step can read.
    """
    s, B, seed = wl.shape, wl.batch, wl.seed
    n = np.full(B, wl.ctx_len, dtype=np.int32) if ctx_len is None else \
        np.asarray(ctx_len, dtype=np.int32)
    taps = normal_bf16(seed, "taps", (B, wl.t_new, s.n_taps * s.hidden), 1.0)
    last = randint(seed, "last_token", (B,), 0, s.vocab)
    cap = wl.cache_cap
    shape = (s.n_layers, B, s.n_kv, cap, s.head_dim)
    nbytes = 2 * np.prod(shape, dtype=np.int64)
    if full_cache is None:
        full_cache = nbytes <= (64 << 20)
    out = dict(taps=taps, last_token=last, ctx_len=n)
    rowlen = cap * s.head_dim
    if full_cache:
        for kv in ("k", "v"):
            c = np.empty(shape, dtype=np.uint16)
            for l in range(s.n_layers):
                for b in range(B):
                    for h in range(s.n_kv):
                        off = (((l * B + b) * s.n_kv) + h) * rowlen
                        c[l, b, h] = normal_bf16(seed, f"{kv}_cache", (cap, s.head_dim), 1.0,
                                                 offset=off)
            out[f"{kv}_cache"] = c
    else:
        for kv in ("k", "v"):
            rows, los = [], []
            for b in range(B):
                lo = max(0, int(n[b]) + wl.t_new - s.window)
                S = int(n[b]) - lo if int(n[b]) > lo else 0
                arr = np.empty((s.n_layers, s.n_kv, S, s.head_dim), dtype=np.uint16)
                for l in range(s.n_layers):
                    for h in range(s.n_kv):
                        off = (((l * B + b) * s.n_kv) + h) * rowlen + lo * s.head_dim
                        arr[l, h] = normal_bf16(seed, f"{kv}_cache", (S, s.head_dim), 1.0,
                                                offset=off)
                rows.append(arr)
                los.append(lo)
            out[f"{kv}_cache"] = WindowCache(rows, los, shape)
    return out


def gemm_inputs(name, N, K, M=8, seed=GEMM_SEED):
    """One matrix of the GEMM microbench: Q4_K weights and bf16 N(0,1) activations."""
    w = q4k_normal(seed, f"gemm.{name}", N, K, 0.02)
    x = normal_bf16(seed, f"gemm.{name}.x", (M, K), 1.0)
    return w, x
