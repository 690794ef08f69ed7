"""The DFlash 2 block-draft forward, step by step, in float64 (test infrastructure only).

Sources (cited per function below):
  [NPU2]  FastFlowLM card "Qwen3.8-27B-DFlash2-NPU2": spec table rows "Draft",
          "Weights", "Taps"; section "How it is used".
  [AIQRE] aiqre page "Qwen3.8-27B-DFlash2": sections "Specification", "Memory".
  [KIT]   Mindket kit page "Qwen3.8-27B-DFlash2-GGUF by z-lab", section
          "For newcomers and experts".
  [MLX]   "Qwen3.8-27B-DFlash2-MLX" card, section "Contents" (the drafter reads
          the target's residual stream at five tapped layers and proposes a whole
          block in one forward).
  [JB]    "Qwen3.8-3.6-27B-blend DFlash2" card: "Model details"; "Quick start"
          (SGLang counts the block of 8, vLLM its 7 proposals).

Steps (the pages leave the wiring of several of them open; each reading taken
here is stated where it is used and listed in the design notes):
  S1  c = RMSNorm(X . W_fc^T), X = the 5 tapped features concatenated in the
      listed layer order                                  [NPU2 "Taps" row]
  S0  block rows: h_0 = E[last token], h_1..7 = shared mask embedding
  per layer (Qwen3-style, [NPU2 "Draft" row]):
      x = RMSNorm(h); Q = x Wq^T; K,V of block rows from x, of context rows from c
      per-head RMSNorm of Q and K, rotary position embedding
      context K,V rows appended to the layer's bf16 cache
      attention of the 8 block queries over (last W cache rows) + (8 block rows)
      two-tap dynamic convolution on the attention output   [NPU2, KIT]
      h += Y Wo^T;  h += (silu(u Wg^T) * (u Wu^T)) Wd^T, u = RMSNorm(h)
  S9  f = RMSNorm(h), block rows 1..7
  S10 logits = f E^T (shared output head), log-softmax, top-K  [NPU2]
"""
import numpy as np

from . import fp8, q4k, q8_0
from .bf16 import bf16_to_f64, f64_to_bf16


# ----------------------------------------------------------------------------
# elementary operations
# ----------------------------------------------------------------------------

def rmsnorm(v, g, eps):
    """Qwen3-style RMSNorm over the last axis: v / sqrt(mean(v^2) + eps) * g."""
    return v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps) * g


def silu(v):
    return v / (1.0 + np.exp(-v))


def rope_inv_freq(d, theta):
    """Rotary frequencies theta^(-2i/d), i = 0..d/2-1 (float64)."""
    i = np.arange(d // 2, dtype=np.float64)
    return theta ** (-2.0 * i / d)


def rope(x, pos, theta):
    """Rotate-half rotary embedding.  x [..., n, d], pos [n] absolute positions.

    Pairs (i, i + d/2) are rotated by angle pos * theta^(-2i/d).
    """
    d = x.shape[-1]
    half = d // 2
    ang = np.asarray(pos, dtype=np.float64)[:, None] * rope_inv_freq(d, theta)[None, :]
    cos, sin = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def softmax(s, axis=-1):
    m = np.max(s, axis=axis, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def logsumexp(s, axis=-1):
    m = np.max(s, axis=axis, keepdims=True)
    return (m + np.log(np.sum(np.exp(s - m), axis=axis, keepdims=True)))[..., 0]


def topk_desc(logits, k):
    """Indices of the k largest values of a 1-D array, ordered by (value desc, index asc)."""
    logits = np.asarray(logits)
    kth = np.partition(logits, logits.size - k)[logits.size - k]   # k-th largest value
    cand = np.flatnonzero(logits >= kth)                           # all ties included
    order = np.lexsort((cand, -logits[cand]))
    return cand[order[:k]]


# ----------------------------------------------------------------------------
# weights
# ----------------------------------------------------------------------------

def dense(w, rows, cols):
    """A linear weight -> float64 [rows, cols].

    w is ("q4k", uint8 bytes), ("q8_0", uint8 bytes), ("fp8", uint8 bytes) or
    ("bf16", uint16 [rows, cols]).
    """
    fmt, data = w
    if fmt == "q4k":
        return q4k.decode_matrix(data, rows, cols)
    if fmt == "q8_0":
        return q8_0.decode_matrix(data, rows, cols)
    if fmt == "fp8":
        return fp8.decode_matrix(data, rows, cols)
    if fmt == "bf16":
        a = np.asarray(data).reshape(rows, cols)
        return bf16_to_f64(a)
    raise ValueError(fmt)


def linear(x, w, rows, cols):
    """y = x . W^T with W [rows=out, cols=in]."""
    return x @ dense(w, rows, cols).T


# ----------------------------------------------------------------------------
# the attention + dynamic convolution block of one layer, one sequence
# ----------------------------------------------------------------------------

def attention(q, kb, vb, kc, vc, n_q, n_kv):
    """Bidirectional block attention with grouped KV heads.

    q [T, n_q, d]; kb, vb [T, n_kv, d] block keys/values; kc, vc [S, n_kv, d]
    cached keys/values in the window.  Every block query sees every key of
    (cache window) + (block rows).  Query head h uses KV head h // (n_q/n_kv).
    Scale 1/sqrt(d), softmax over keys.  Returns o [T, n_q, d].
    """
    T, _, d = q.shape
    G = n_q // n_kv
    keys = np.concatenate([kc, kb], axis=0)       # [S+T, n_kv, d]
    vals = np.concatenate([vc, vb], axis=0)
    o = np.empty_like(q)
    for h in range(n_q):
        g = h // G
        s = q[:, h, :] @ keys[:, g, :].T / np.sqrt(d)   # [T, S+T]
        o[:, h, :] = softmax(s, axis=-1) @ vals[:, g, :]
    return o


def dynamic_conv(o, w_conv):
    """Two-tap dynamic convolution along the block.

    o [T, n_q, d] attention output; w_conv [2 n_q, n_q d] (float64).
    z_t = W_c . vec(o_t);  a_{t,h} = z_t[h], b_{t,h} = z_t[n_q + h];
    y_{t,h} = a_{t,h} * o_{t,h} + b_{t,h} * o_{t-1,h},  o_{-1} = 0.
    The pages say the convolutions sit inside the backbone and keep draft quality
    from dropping along the block; this per-head, input-dependent two-tap form
    is the reading used here.  Returns y [T, n_q, d].
    """
    T, n_q, d = o.shape
    z = o.reshape(T, n_q * d) @ w_conv.T           # [T, 2 n_q]
    a, b = z[:, :n_q], z[:, n_q:]
    prev = np.concatenate([np.zeros((1, n_q, d)), o[:-1]], axis=0)
    return a[:, :, None] * o + b[:, :, None] * prev


# ----------------------------------------------------------------------------
# the whole step
# ----------------------------------------------------------------------------

def draft_step(cfg, W, taps, last_token, ctx_len, k_cache, v_cache, want_logits=True):
    """One block-draft forward for a batch of independent sequences.

    cfg: dict with n_layers, hidden, ffn, n_q, n_kv, head_dim, window, vocab,
         n_taps, block, top_k, rms_eps, rope_theta.
    W:   dict of weights.  Linear weights are ("q4k", "q8_0" or "fp8", bytes) or ("bf16", u16):
         fc [H, n_taps H], and per layer l: wq [n_q d, H], wk/wv [n_kv d, H],
         wo [H, n_q d], wg/wu [F, H], wd [H, F].  bf16 uint16 arrays: hidden_norm,
         final_norm [H], mask_emb [H], embed [V, H], lm_head [V, H], and per layer
         in_norm, post_norm [H], q_norm, k_norm [d], w_conv [2 n_q, n_q d].
         Layer l entries are keyed "l{l}.<name>".
    taps [B, T_new, n_taps H] bf16; last_token [B]; ctx_len [B] (rows already
    cached before this step); k_cache/v_cache: indexable as [l, b, kvh, rows, :]
    (bf16 uint16), holding at least the window rows before the step.

    Returns a dict:
      hidden  [L+1, B, T, H]  h after block assembly and after each layer
      fused   [B, T_new, H]   the fused tap rows c
      new_k, new_v [L, B, n_kv, T_new, d] bf16 rows written at ctx_len..+T_new-1
      logits  [B, T-1, V]     (if want_logits)
      lse     [B, T-1]
      cand_ids [B, T-1, K], cand_logp [B, T-1, K]
    """
    L, H, F = cfg["n_layers"], cfg["hidden"], cfg["ffn"]
    n_q, n_kv, d = cfg["n_q"], cfg["n_kv"], cfg["head_dim"]
    Wn, V, nt = cfg["window"], cfg["vocab"], cfg["n_taps"]
    T, K, eps, theta = cfg["block"], cfg["top_k"], cfg["rms_eps"], cfg["rope_theta"]
    taps = np.asarray(taps)
    B, T_new, _ = taps.shape
    g = lambda name: bf16_to_f64(np.asarray(W[name]))

    # S1: fuse the five tapped target features (in listed layer order) with fc
    X = bf16_to_f64(taps).reshape(B * T_new, nt * H)
    c = rmsnorm(linear(X, W["fc"], H, nt * H), g("hidden_norm"), eps).reshape(B, T_new, H)

    # S0: block assembly: anchor = embedding of the last accepted token, then mask rows
    E = np.asarray(W["embed"])
    h = np.empty((B, T, H))
    h[:, 0, :] = bf16_to_f64(E[np.asarray(last_token)])
    h[:, 1:, :] = g("mask_emb")[None, None, :]

    hidden = [h.copy()]
    new_k = np.empty((L, B, n_kv, T_new, d), dtype=np.uint16)
    new_v = np.empty((L, B, n_kv, T_new, d), dtype=np.uint16)
    for l in range(L):
        p = f"l{l}."
        x = rmsnorm(h, g(p + "in_norm"), eps)                         # [B, T, H]
        q = linear(x.reshape(B * T, H), W[p + "wq"], n_q * d, H).reshape(B, T, n_q, d)
        xc = np.concatenate([x.reshape(B * T, H), c.reshape(B * T_new, H)], axis=0)
        kk = linear(xc, W[p + "wk"], n_kv * d, H)
        vv = linear(xc, W[p + "wv"], n_kv * d, H)
        kb = kk[:B * T].reshape(B, T, n_kv, d)
        vb = vv[:B * T].reshape(B, T, n_kv, d)
        kc_new = kk[B * T:].reshape(B, T_new, n_kv, d)
        vc_new = vv[B * T:].reshape(B, T_new, n_kv, d)
        q = rmsnorm(q, g(p + "q_norm"), eps)
        kb = rmsnorm(kb, g(p + "k_norm"), eps)
        kc_new = rmsnorm(kc_new, g(p + "k_norm"), eps)
        wconv = g(p + "w_conv")
        y = np.empty((B, T, n_q, d))
        for b in range(B):
            n = int(ctx_len[b])
            pos_blk = n + T_new + np.arange(T)
            pos_ctx = n + np.arange(T_new)
            qb = rope(q[b].transpose(1, 0, 2), pos_blk, theta).transpose(1, 0, 2)
            kbb = rope(kb[b].transpose(1, 0, 2), pos_blk, theta).transpose(1, 0, 2)
            kcn = rope(kc_new[b].transpose(1, 0, 2), pos_ctx, theta)   # [n_kv, T_new, d]
            # the cache stores bf16: the appended rows are rounded when written
            new_k[l, b] = f64_to_bf16(kcn)
            new_v[l, b] = f64_to_bf16(vc_new[b].transpose(1, 0, 2))
            lo = max(0, n + T_new - Wn)
            # window rows: old cache rows [lo, n) followed by the appended rows
            old_lo = lo
            kc_old = bf16_to_f64(np.asarray(k_cache[l, b, :, old_lo:n, :]))  # [n_kv, S, d]
            vc_old = bf16_to_f64(np.asarray(v_cache[l, b, :, old_lo:n, :]))
            new_lo = max(0, lo - n)
            kc_win = np.concatenate([kc_old, bf16_to_f64(new_k[l, b])[:, new_lo:]], axis=1)
            vc_win = np.concatenate([vc_old, bf16_to_f64(new_v[l, b])[:, new_lo:]], axis=1)
            o = attention(qb, kbb, vb[b], kc_win.transpose(1, 0, 2),
                          vc_win.transpose(1, 0, 2), n_q, n_kv)
            y[b] = dynamic_conv(o, wconv)
        h = h + linear(y.reshape(B * T, n_q * d), W[p + "wo"], H, n_q * d).reshape(B, T, H)
        u = rmsnorm(h, g(p + "post_norm"), eps).reshape(B * T, H)
        mid = silu(linear(u, W[p + "wg"], F, H)) * linear(u, W[p + "wu"], F, H)
        h = h + linear(mid, W[p + "wd"], H, F).reshape(B, T, H)
        hidden.append(h.copy())

    # S9: final norm on the proposal rows 1..T-1 (row 0 is the anchor)
    f = rmsnorm(h[:, 1:, :], g("final_norm"), eps)                  # [B, T-1, H]
    out = dict(hidden=np.stack(hidden), fused=c, new_k=new_k, new_v=new_v, final=f)
    out.update(lm_head_topk(f, W["lm_head"], K, want_logits=want_logits))
    return out


def lm_head_topk(f, lm_head, K, want_logits=True, chunk=16384):
    """S10: logits = f E^T with the shared output head, log-softmax, top-K.

    f [B, P, H] float64; lm_head bf16 [V, H].  Candidates are ordered by (logit
    desc, id asc); cand_logp = logit - logsumexp(logits).  Processed in vocabulary
    chunks so the float64 copy of the head stays bounded.
    """
    E = np.asarray(lm_head)
    V, H = E.shape
    B, P, _ = f.shape
    fr = f.reshape(B * P, H)
    logits = np.empty((B * P, V))
    for v0 in range(0, V, chunk):
        v1 = min(V, v0 + chunk)
        logits[:, v0:v1] = fr @ bf16_to_f64(E[v0:v1]).T
    lse = logsumexp(logits, axis=-1)
    ids = np.stack([topk_desc(logits[i], K) for i in range(B * P)])
    lp = np.take_along_axis(logits, ids, axis=-1) - lse[:, None]
    res = dict(lse=lse.reshape(B, P), cand_ids=ids.reshape(B, P, K).astype(np.int32),
               cand_logp=lp.reshape(B, P, K))
    if want_logits:
        res["logits"] = logits.reshape(B, P, V)
    return res
