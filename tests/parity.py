"""Comparison helpers between the GPU library and the oracle (test infrastructure)."""
import dataclasses

import numpy as np

from block_diffusion_draft_amd import synth
from oracle import draft as odraft
from oracle import select as oselect
from oracle.bf16 import bf16_to_f64

# Tolerances for the bf16-activation GPU path against the float64 oracle
HIDDEN_REL_L2 = 2e-2        # per layer, per sequence
LOGIT_MAX_ABS = 5e-2
TOPK_BAND = 2 * LOGIT_MAX_ABS
PATH_MARGIN = 1e-4


def subset_inputs(wl, inputs, seqs):
    """Inputs of the sequences `seqs` only (sequences are independent)."""
    out = {k: inputs[k][seqs] for k in ("taps", "last_token", "ctx_len")}
    for c in ("k_cache", "v_cache"):
        v = inputs[c]
        if isinstance(v, np.ndarray):
            out[c] = v[:, seqs]
        else:
            out[c] = synth.WindowCache([v.rows[b] for b in seqs], [v.lo[b] for b in seqs],
                                       v.shape)
    return out


def run_oracle(wl, W, inputs, seqs=None, want_logits=True):
    if seqs is not None:
        inputs = subset_inputs(wl, inputs, seqs)
    return odraft.draft_step(wl.shape.as_dict(), W, inputs["taps"], inputs["last_token"],
                             inputs["ctx_len"], inputs["k_cache"], inputs["v_cache"],
                             want_logits=want_logits)


def run_oracle_chunked(wl, W, inputs, chunk=8, say=print):
    """The oracle over every sequence, `chunk` sequences per call (a progress line per
    call); the per-sequence outputs concatenated along the batch axis."""
    parts = []
    for b0 in range(0, wl.batch, chunk):
        seqs = list(range(b0, min(wl.batch, b0 + chunk)))
        say(f"  oracle: sequences {seqs[0]}..{seqs[-1]} of {wl.batch}")
        parts.append(run_oracle(wl, W, inputs, seqs=seqs))
    out = {}
    for k, v in parts[0].items():
        axis = 1 if k in ("hidden", "new_k", "new_v") else 0
        out[k] = np.concatenate([p[k] for p in parts], axis=axis)
    return out


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def check_hidden(gpu_hidden, ref_hidden, tol=HIDDEN_REL_L2):
    """gpu_hidden, ref_hidden [L+1, B, T, H]; returns the worst rel L2."""
    worst = 0.0
    for l in range(ref_hidden.shape[0]):
        for b in range(ref_hidden.shape[1]):
            r = rel_l2(gpu_hidden[l, b], ref_hidden[l, b])
            assert r <= tol, (l, b, r)
            worst = max(worst, r)
    return worst


def check_topk_reanchored(gpu_logits, gpu_ids, gpu_lp, K):
    """The GPU's candidates from its own fp32 logits: ids exactly, log-probs to fp32."""
    B, P, V = gpu_logits.shape
    lg = gpu_logits.astype(np.float64)
    for b in range(B):
        for t in range(P):
            ids = odraft.topk_desc(lg[b, t], K)
            assert np.array_equal(ids, gpu_ids[b, t]), (b, t, ids, gpu_ids[b, t])
            lse = odraft.logsumexp(lg[b, t])
            assert np.allclose(gpu_lp[b, t], lg[b, t, ids] - lse, rtol=0, atol=2e-5)


def check_topk_valid(ref_logits, gpu_ids, K, band=TOPK_BAND):
    """End to end: every id well above the oracle's K-th logit is chosen, and every
    chosen id is at most `band` below it.  Returns the number of rows whose set
    differs from the oracle's (all of them within the band)."""
    B, P, V = ref_logits.shape
    differ = 0
    for b in range(B):
        for t in range(P):
            row = ref_logits[b, t]
            ref = odraft.topk_desc(row, K)
            lk = row[ref[-1]]
            must = np.flatnonzero(row > lk + band)
            got = set(int(i) for i in gpu_ids[b, t])
            assert set(must.tolist()) <= got, (b, t)
            assert all(row[i] >= lk - band for i in got), (b, t)
            differ += set(ref.tolist()) != got
    return differ


def check_paths(gpu_ids, gpu_lp, gpu_draft, code_a, code_b, s):
    """The GPU path equals the Viterbi path over the GPU's own candidates (same
    fp32 precision); a different path is accepted only at a near tie."""
    A = bf16_to_f64(code_a)
    Bm = bf16_to_f64(code_b)
    ties = 0
    for b in range(gpu_ids.shape[0]):
        ids = gpu_ids[b]
        T32 = oselect.pair_scores(ids, A.astype(np.float32), Bm.astype(np.float32), s,
                                  dtype=np.float32)
        path, _ = oselect.viterbi(gpu_lp[b].astype(np.float32), T32, dtype=np.float32)
        want = ids[np.arange(ids.shape[0]), path]
        if np.array_equal(want, gpu_draft[b]):
            continue
        # near tie: compare exact scores of both paths
        T64 = oselect.pair_scores(ids, A, Bm, s)
        gp = np.array([list(ids[t]).index(gpu_draft[b, t]) for t in range(ids.shape[0])])
        best64, _ = oselect.viterbi(gpu_lp[b].astype(np.float64), T64)
        m = oselect.path_score(gpu_lp[b], T64, best64) - oselect.path_score(gpu_lp[b], T64, gp)
        assert m < PATH_MARGIN, (b, m)
        ties += 1
    return ties


def with_shape(wl, **kw):
    return dataclasses.replace(wl, shape=dataclasses.replace(wl.shape, **kw))
