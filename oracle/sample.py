"""Sampled acceptance of a drafted block by exact rejection sampling (test infrastructure only).

Sources: Mindket kit page "Qwen3.8-27B-DFlash2-GGUF by z-lab", section "For newcomers
and experts" (the card's claim that sampling keeps the target's output distribution)
and section "Good to know" (sampler settings: temperature 1.0, top-p 0.95, top-k 20);
aiqre model page "Qwen3.8-27B-DFlash2", "Overview" (faithful sampling); JetBrains card
"Qwen3.8-3.6-27B-blend DFlash2", "Quick start" (the same settings for API requests and
the MLX runner).

The pages give the sampler settings and the guarantee, not the procedure.  Readings:
  * Target distribution at block position j: logits divided by the temperature; keep
    the top_k largest (ties: lowest token id first); softmax over those; order them by
    (probability desc, id asc) and keep each token while the mass of the tokens before
    it is below top_p (the smallest prefix whose mass reaches top_p); renormalise.
  * The draft's proposals are a deterministic function of the context (the selector's
    path), so the proposal distribution at position j is a point mass on x_j.
    Rejection sampling against that proposal: accept x_j when u < p_j(x_j); on
    rejection emit a token drawn from p_j with x_j removed and the rest renormalised,
    and stop; when all n proposals are accepted, emit a token drawn from p_n.  Every
    emitted token then has the target's distribution given the tokens before it.
  * The random numbers are inputs: u[b, j, 0] is position j's acceptance draw,
    u[b, j, 1] its sampling draw (the residual at j < n, the bonus token at j = n).
    A draw takes the first token, in (probability desc, id asc) order, whose cumulative
    weight exceeds u times the total weight.

Every function also reports a margin: the smallest distance, relative to the mass
involved, between a number this computation compared and the threshold it was
compared with.  A float32 implementation can take another branch only where that
margin is of the order of float32 rounding.
"""
import numpy as np


def target_dist(logits, temperature, top_k, top_p):
    """One row of target logits [V] -> (ids [m], probs [m], margin).

    ids in (probability desc, id asc) order; probs sum to 1 over the kept set.
    """
    z = np.asarray(logits, dtype=np.float64) / float(temperature)
    V = z.shape[0]
    order = np.lexsort((np.arange(V), -z))[:top_k]      # logit desc, then id asc
    w = np.exp(z[order] - z[order[0]])
    p = w / w.sum()
    before = np.concatenate(([0.0], np.cumsum(p)[:-1]))  # mass of the tokens before each
    keep = before < top_p
    m = int(keep.sum())
    margin = np.inf
    if top_p < 1.0:
        margin = top_p - before[m - 1]
        if m < len(p):
            margin = min(margin, before[m] - top_p)
    q = p[:m] / p[:m].sum()
    return order[:m].astype(np.int64), q, margin


def draw(weights, u):
    """Index of the first entry whose cumulative weight exceeds u * sum(weights), and the
    margin of that choice relative to the total."""
    w = np.asarray(weights, dtype=np.float64)
    total = w.sum()
    t = u * total
    cum = np.cumsum(w)
    c = int(np.searchsorted(cum, t, side="right"))
    c = min(c, len(w) - 1)
    lo = cum[c - 1] if c > 0 else 0.0
    margin = min(cum[c] - t, t - lo) / total
    return c, margin


def accept_sequence(draft, dists, u):
    """One sequence: draft [n] token ids, dists = n + 1 (ids, probs) pairs, u [n + 1, 2]
    -> (accept_len k, out [n + 1] with draft[:k], the emitted token, then -1, margin)."""
    n = len(draft)
    out = np.full(n + 1, -1, dtype=np.int64)
    margin = np.inf
    for j in range(n + 1):
        ids, probs = dists[j]
        if j == n:
            c, mg = draw(probs, u[j, 1])
            out[j] = ids[c]
            return n, out, min(margin, mg)
        x = int(draft[j])
        hit = np.nonzero(ids == x)[0]
        px = probs[hit[0]] if len(hit) else 0.0
        margin = min(margin, abs(u[j, 0] - px))
        if u[j, 0] < px:
            out[j] = x
            continue
        rest = ids != x
        c, mg = draw(probs[rest], u[j, 1])
        out[j] = ids[rest][c]
        return j, out, min(margin, mg)


def verify_sampled(draft, logits, u, temperature, top_k, top_p):
    """draft int [B, n], logits [B, n + 1, V], u [B, n + 1, 2]
    -> (accept_len [B], out [B, n + 1] (-1 padded), margin [B])."""
    draft = np.asarray(draft)
    logits = np.asarray(logits)
    u = np.asarray(u, dtype=np.float64)
    B, n = draft.shape
    assert logits.shape[:2] == (B, n + 1) and u.shape == (B, n + 1, 2)
    acc = np.zeros(B, dtype=np.int32)
    out = np.full((B, n + 1), -1, dtype=np.int32)
    margin = np.full(B, np.inf)
    for b in range(B):
        dists, cut = [], []
        for j in range(n + 1):
            ids, probs, m = target_dist(logits[b, j], temperature, top_k, top_p)
            dists.append((ids, probs))
            cut.append(m)
        k, o, m2 = accept_sequence(draft[b], dists, u[b])
        # the top-p cuts of the positions the procedure looked at, 0 .. k
        acc[b], out[b], margin[b] = k, o, min(min(cut[:k + 1]), m2)
    return acc, out, margin
