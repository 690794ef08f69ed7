"""Invariants of the composed draft step (CPU).

The pages print no worked example of the composed forward (taps -> layers ->
logits), so its composition is "parity unpinned" beyond the pinned components;
these tests check properties that hold by construction of the method.
"""
import dataclasses

import numpy as np

from block_diffusion_draft_amd import synth
from oracle import draft


def run(wl, W=None, inp=None, **kw):
    s = wl.shape
    W = W if W is not None else synth.make_weights(s, wl.seed)
    inp = inp if inp is not None else synth.make_step_inputs(wl)
    out = draft.draft_step(s.as_dict(), W, inp["taps"], inp["last_token"], inp["ctx_len"],
                           inp["k_cache"], inp["v_cache"], **kw)
    return out, W, inp


def test_shapes_and_block_accounting():
    """Block of 8 = 1 anchor + 7 proposals (JetBrains card "Quick start": SGLang
    counts 8, vLLM 7); top-K ids distinct and sorted by log-prob."""
    wl = synth.WORKLOADS["tiny"]
    out, W, inp = run(wl)
    s = wl.shape
    assert out["hidden"].shape == (s.n_layers + 1, 1, 8, s.hidden)
    assert out["cand_ids"].shape == (1, 7, s.top_k)
    assert out["logits"].shape == (1, 7, s.vocab)
    lp = out["cand_logp"][0]
    assert np.all(np.diff(lp, axis=1) <= 0) and np.all(lp < 0)
    for t in range(7):
        assert len(set(out["cand_ids"][0, t])) == s.top_k


def test_rows_outside_window_are_never_read():
    """Poisoning every cache row outside the attention window changes nothing."""
    wl = dataclasses.replace(synth.WORKLOADS["tiny"], cache_extra=5)
    out, W, inp = run(wl)
    n, T_new, Wn = wl.ctx_len, wl.t_new, wl.shape.window
    lo = n + T_new - Wn
    for c in ("k_cache", "v_cache"):
        inp[c][:, :, :, :lo, :] = 0x7FC0        # bf16 NaN
        inp[c][:, :, :, n:, :] = 0x7FC0         # rows the step overwrites / spare rows
    out2, _, _ = run(wl, W, inp)
    assert np.isfinite(out2["logits"]).all()
    assert np.array_equal(out["logits"], out2["logits"])


def test_window_rows_order_does_not_matter():
    """Attention is a set operation over the keys: permuting the cached window rows
    (keys and values together) leaves the output unchanged up to rounding."""
    wl = synth.WORKLOADS["tiny"]
    out, W, inp = run(wl)
    n, T_new, Wn = wl.ctx_len, wl.t_new, wl.shape.window
    lo = n + T_new - Wn
    perm = np.random.default_rng(0).permutation(np.arange(lo, n))
    for c in ("k_cache", "v_cache"):
        inp[c][:, :, :, lo:n, :] = inp[c][:, :, :, perm, :]
    out2, _, _ = run(wl, W, inp)
    assert np.allclose(out["logits"], out2["logits"], rtol=1e-9, atol=1e-12)


def test_no_context_rows_makes_taps_irrelevant():
    """With a window that admits no cache row, the fused taps (which enter only as
    context K/V rows) cannot influence the block."""
    wl = synth.WORKLOADS["tiny"]
    s0 = dataclasses.replace(wl.shape, window=0)
    wl0 = dataclasses.replace(wl, shape=s0)
    out, W, inp = run(wl0)
    inp["taps"] = synth.normal_bf16(99, "other", inp["taps"].shape, 1.0)
    out2, _, _ = run(wl0, W, inp)
    assert np.array_equal(out["logits"], out2["logits"])


def test_taps_matter_with_a_window():
    wl = synth.WORKLOADS["tiny"]
    out, W, inp = run(wl)
    inp["taps"] = synth.normal_bf16(99, "other", inp["taps"].shape, 1.0)
    out2, _, _ = run(wl, W, inp)
    assert not np.allclose(out["logits"], out2["logits"])


def test_appended_rows_are_bf16_of_the_roped_keys():
    """The appended cache rows are the context keys after k-norm and RoPE,
    stored in bf16; position n + i for context row i."""
    wl = synth.WORKLOADS["tiny"]
    out, W, inp = run(wl)
    s = wl.shape
    k = out["new_k"][0, 0]                     # [n_kv, T_new, d]
    from oracle.bf16 import bf16_to_f64
    kk = bf16_to_f64(k)
    # rope preserves norms; k-norm with unit gain gives rms 1 per head -> |k| = sqrt(d)
    assert np.allclose(np.linalg.norm(kk, axis=-1), np.sqrt(s.head_dim), rtol=1e-2)


def test_full_window_when_context_is_short():
    """W >= n + T_new: every cached row is attended (same result as a huge window)."""
    wl = synth.WORKLOADS["tiny"]
    sA = dataclasses.replace(wl.shape, window=wl.ctx_len + wl.t_new)
    sB = dataclasses.replace(wl.shape, window=10 ** 6)
    outA, W, inp = run(dataclasses.replace(wl, shape=sA))
    outB, _, _ = run(dataclasses.replace(wl, shape=sB), W, inp)
    assert np.array_equal(outA["logits"], outB["logits"])
