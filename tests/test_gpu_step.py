"""GPU parity of the whole draft step against the float64 oracle.

Bars: per-layer hidden-state relative L2 <= 2e-2 and logits max-abs <= 5e-2
(bf16 activations vs float64); top-K ids exact when re-anchored on the GPU's own
logits and valid within a 0.1 band against the oracle's; the path equal to the
Viterbi path over the GPU's own candidates (near ties aside); appended cache
rows within bf16 rounding; prefix acceptance exact; two runs bitwise equal.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

from block_diffusion_draft_amd import runner, synth
from oracle.bf16 import bf16_to_f64
from oracle.verify import verify_prefix
from tests import parity

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_outputs(bufs):
    torch.cuda.synchronize()
    return dict(hidden=bufs.dbg_hidden.cpu().numpy().astype(np.float64),
                logits=bufs.dbg_logits.cpu().numpy(),
                ids=bufs.cand_ids.cpu().numpy(),
                lp=bufs.cand_logp.cpu().numpy(),
                draft=bufs.draft.cpu().numpy())


def full_check(wl, bufs, ref, seqs=None):
    g = gpu_outputs(bufs)
    if seqs is not None:
        for k in ("hidden",):
            g[k] = g[k][:, seqs]
        for k in ("logits", "ids", "lp", "draft"):
            g[k] = g[k][seqs]
    worst = parity.check_hidden(g["hidden"], ref["hidden"])
    dl = np.abs(g["logits"] - ref["logits"]).max()
    assert dl <= parity.LOGIT_MAX_ABS, dl
    parity.check_topk_reanchored(g["logits"], g["ids"], g["lp"], wl.shape.top_k)
    differ = parity.check_topk_valid(ref["logits"], g["ids"], wl.shape.top_k)
    W = bufs.host_W
    ties = parity.check_paths(g["ids"], g["lp"], g["draft"], W["code_a"], W["code_b"],
                              wl.shape.pair_scale)
    for which, key in (("k", "new_k"), ("v", "new_v")):
        got = bf16_to_f64(bufs.new_rows(which))
        if seqs is not None:
            got = got[:, seqs]
        want = bf16_to_f64(ref[key])
        assert np.allclose(got, want, rtol=2 ** -7, atol=2e-2), which
    say(f"  hidden worst rel L2 {worst:.2e}, logits max-abs {dl:.2e}, "
        f"top-K rows differing within band {differ}, path near-ties {ties}")
    return g


def check_verify(bufs, g):
    P = g["draft"].shape[1]
    B = g["draft"].shape[0]
    for k in range(P + 1):
        tgt = np.zeros((B, P + 1), dtype=np.int32)
        tgt[:, :k] = g["draft"][:, :k]
        if k < P:
            tgt[:, k] = g["draft"][:, k] + 1
        tgt[:, k + 1:] = 7
        bufs.verify(torch.from_numpy(tgt).cuda())
        torch.cuda.synchronize()
        ra, ro = verify_prefix(g["draft"], tgt)
        assert np.array_equal(bufs.accept_len.cpu().numpy(), ra)
        assert np.array_equal(bufs.out_tokens.cpu().numpy(), ro)


def test_tiny_step_parity_and_determinism():
    wl = synth.WORKLOADS["tiny"]
    say(f"[step] {wl.name}")
    bufs = runner.StepBuffers(wl)
    bufs.step()
    ref = parity.run_oracle(wl, bufs.host_W, bufs.inputs)
    g = full_check(wl, bufs, ref)
    check_verify(bufs, g)
    first = {k: v.copy() for k, v in g.items()}
    bufs.step()
    g2 = gpu_outputs(bufs)
    for k in first:
        assert np.array_equal(first[k], g2[k]), k


def test_tiny_step_gain_path_and_batch():
    """Norm gains 1 + 0.1 N(0,1), 3 sequences with different context lengths
    (one shorter than the window, one whose window starts mid-cache)."""
    wl = dataclasses.replace(synth.WORKLOADS["tiny"], batch=3, seed=11, cache_extra=4)
    say(f"[step] tiny gains, batch 3")
    W = synth.make_weights(wl.shape, wl.seed, gain_jitter=0.1)
    inputs = synth.make_step_inputs(wl, ctx_len=[48, 10, 0])
    bufs = runner.StepBuffers(wl, weights=W, inputs=inputs)
    bufs.step()
    ref = parity.run_oracle(wl, W, inputs)
    full_check(wl, bufs, ref)


def test_tiny_step_short_tnew():
    wl = dataclasses.replace(synth.WORKLOADS["tiny"], t_new=3, seed=12)
    say("[step] tiny t_new=3")
    bufs = runner.StepBuffers(wl)
    bufs.step()
    full_check(wl, bufs, parity.run_oracle(wl, bufs.host_W, bufs.inputs))


def test_tiny_step_invalid_sequence_is_skipped():
    """ctx_len out of range for one sequence: its outputs are -1 / -inf, the
    others are unaffected, and no cache row of it is written."""
    wl = dataclasses.replace(synth.WORKLOADS["tiny"], batch=2, seed=13)
    say("[step] tiny invalid sequence")
    good = runner.StepBuffers(wl)
    good.step()
    g_ok = gpu_outputs(good)
    inputs = dict(good.inputs)
    inputs["ctx_len"] = np.array([48, 10 ** 6], dtype=np.int32)
    bad = runner.StepBuffers(wl, weights=good.host_W, inputs=inputs)
    kc_before = bad.k_cache.clone()
    bad.step()
    g = gpu_outputs(bad)
    assert np.array_equal(g["draft"][1], [-1] * 7)
    assert (g["ids"][1] == -1).all() and np.isneginf(g["lp"][1]).all()
    assert np.array_equal(g["draft"][0], g_ok["draft"][0])
    assert np.array_equal(g["logits"][0], g_ok["logits"][0])
    assert torch.equal(bad.k_cache[:, 1], kc_before[:, 1])


def test_tiny_step_rows_outside_window_unread():
    """NaN in every cache row outside the window leaves the outputs finite and
    bitwise equal to a run with finite data there."""
    wl = dataclasses.replace(synth.WORKLOADS["tiny"], seed=14, cache_extra=6)
    say("[step] tiny poison")
    a = runner.StepBuffers(wl)
    a.step()
    ga = gpu_outputs(a)
    inp = dict(a.inputs)
    n, T_new, Wn = wl.ctx_len, wl.t_new, wl.shape.window
    lo = n + T_new - Wn
    for c in ("k_cache", "v_cache"):
        arr = inp[c].copy()
        arr[:, :, :, :lo, :] = runner.BF16_NAN
        arr[:, :, :, n + T_new:, :] = runner.BF16_NAN
        inp[c] = arr
    b = runner.StepBuffers(wl, weights=a.host_W, inputs=inp)
    b.step()
    gb = gpu_outputs(b)
    assert np.isfinite(gb["logits"]).all()
    for k in ga:
        assert np.array_equal(ga[k], gb[k]), k


@pytest.mark.timeout(900)
def test_full_step_b1_parity():
    """The pages' draft shape, one sequence, 4096 cached rows."""
    wl = synth.WORKLOADS["full_b1"]
    say(f"[step] {wl.name}: generating inputs")
    bufs = runner.StepBuffers(wl)
    say("  running GPU step")
    bufs.step()
    torch.cuda.synchronize()
    say("  running oracle")
    ref = parity.run_oracle(wl, bufs.host_W, bufs.inputs)
    g = full_check(wl, bufs, ref)
    check_verify(bufs, g)
    # the same step with N(0, 1) selector codebooks: the pair term ~ N(0, 1) decides
    # the path (top 16, rank 256); it must be the float64 Viterbi path over the GPU's
    # own candidates and differ from the per-position argmax
    from tests.test_gpu_select import path_checks
    ca, cb = synth.selector_codebooks(wl.shape, wl.seed + 1000, std=1.0)
    bufs.dw.tensors["code_a"].copy_(torch.from_numpy(ca.view(np.int16)))
    bufs.dw.tensors["code_b"].copy_(torch.from_numpy(cb.view(np.int16)))
    bufs.step(dbg=False)
    torch.cuda.synchronize()
    ids, lp = bufs.cand_ids.cpu().numpy(), bufs.cand_logp.cpu().numpy()
    draft = bufs.draft.cpu().numpy()
    assert np.array_equal(ids, g["ids"])              # candidates do not depend on codebooks
    nonarg = path_checks(ids, lp, draft, ca, cb, wl.shape.pair_scale, brute=False)
    say(f"  N(0, 1) codebooks: path {draft[0].tolist()} (argmax path "
        f"{ids[0, :, 0].tolist()})")
    assert nonarg == 1


def test_tiny_step_tied_logits_take_lowest_ids():
    """Every output-head row equal: all logits of a row tie, more of them reach the
    selection threshold than the candidate list holds, and the exact fallback scan
    must return ids 0..K-1 (ties broken by id) with log-prob -log(V)."""
    wl = dataclasses.replace(synth.WORKLOADS["tiny"], seed=15)
    say("[step] tiny tied logits")
    W = synth.make_weights(wl.shape, wl.seed)
    E = np.repeat(W["embed"][:1], wl.shape.vocab, axis=0)
    W["embed"] = E
    W["lm_head"] = E
    bufs = runner.StepBuffers(wl, weights=W)
    bufs.step()
    g = gpu_outputs(bufs)
    K, V = wl.shape.top_k, wl.shape.vocab
    assert (g["ids"] == np.arange(K)).all()
    assert np.allclose(g["lp"], -np.log(V), atol=1e-4)
    ref = parity.run_oracle(wl, W, bufs.inputs)
    assert (ref["cand_ids"] == np.arange(K)).all()


@pytest.mark.parametrize("block,batch", [(5, 2), (4, 1), (4, 2), (2, 3)])
def test_tiny_step_block_lengths(block, batch):
    """Shorter blocks (P = block - 1 proposals; the pages' MLX example drafts with a
    block of 5): block 5 x 2 sequences runs the MLP products over 20 rows (row-tiled
    kernel); block 4 x 1 and x 2 make the (hi, lo) row pairs 4 and 8 rows apart (added
    inside the streaming kernel); block 2 leaves one proposal per sequence."""
    shape = dataclasses.replace(synth.TINY, block=block)
    wl = dataclasses.replace(synth.WORKLOADS["tiny"], shape=shape, batch=batch, seed=20 + block)
    say(f"[step] tiny block {block}, batch {batch}")
    bufs = runner.StepBuffers(wl)
    bufs.step()
    ref = parity.run_oracle(wl, bufs.host_W, bufs.inputs)
    g = full_check(wl, bufs, ref)
    assert g["draft"].shape == (batch, block - 1)
    check_verify(bufs, g)


@pytest.mark.parametrize("fmt,head_dim,batch", [("q4k", 128, 1), ("q4k", 128, 2), ("q4k", 64, 1),
                                                ("q8_0", 64, 2)])
def test_mid_step_streaming_products(fmt, head_dim, batch):
    """A 2-layer drafter (hidden 1024) whose products all have K a multiple of 1024, so
    at 8 and 16 rows they run on the 16-row streaming kernels (Q4_K and Q8_0), with the
    (hi, lo) pair added in-kernel; heads of 128 and of 64."""
    n_q = 1024 // head_dim
    s = dataclasses.replace(synth.MID, weight_fmt=fmt, head_dim=head_dim, n_q=n_q,
                            n_kv=n_q // 4)
    wl = dataclasses.replace(synth.WORKLOADS["tiny"], shape=s, batch=batch, ctx_len=96,
                             seed=50 + batch + head_dim)
    say(f"[step] mid {fmt} head_dim {head_dim} batch {batch}")
    bufs = runner.StepBuffers(wl)
    bufs.step()
    torch.cuda.synchronize()
    ref = parity.run_oracle(wl, bufs.host_W, bufs.inputs)
    g = full_check(wl, bufs, ref)
    check_verify(bufs, g)


@pytest.mark.parametrize("fmt,batch,vocab", [("q4k", 4, 0), ("q8_0", 4, 0), ("bf16", 4, 0),
                                             ("q4k", 8, 0), ("q8_0", 16, 0),
                                             ("q4k", 128, 0), ("fp8", 128, 0),
                                             ("bf16", 128, 16 * 4133),
                                             ("bf16", 16, 16 * 8229)])
def test_mid_step_many_rows(fmt, batch, vocab):
    """Many sequences of a 2-layer drafter: every product has more than 16 rows and runs
    on the many-row GEMM with the format's weight decode.  4 sequences: 32 block rows, 64
    with the context rows or the (hi, lo) pairs, split-K where the tiles are few, the
    output head (28 rows) with the deferred final norm in its epilogue.  8 and 16
    sequences (quantised): the MLP products are one 128- or 256-row tile of 64 or 128
    rows and their lo rows, which the kernel adds itself (partials of half the rows).
    128 sequences:
    1024 block rows over 4 row tiles, 2048 MLP rows over 8, the 896-row head, and (bf16)
    a vocabulary of 4133 16-column tiles whose last 256-column head tile is ragged.  16
    sequences, bf16, a vocabulary of 8229 16-column tiles: the 112-row head on 128 x 512
    tiles (258 of them, the last ragged) with 64-deep operand stages."""
    s = dataclasses.replace(synth.MID, weight_fmt=fmt)
    if vocab:
        s = dataclasses.replace(s, vocab=vocab)
    wl = dataclasses.replace(synth.WORKLOADS["tiny"], shape=s, batch=batch, ctx_len=96, seed=61)
    say(f"[step] mid {fmt} batch {batch}, vocab {s.vocab}")
    bufs = runner.StepBuffers(wl)
    bufs.step()
    torch.cuda.synchronize()
    ref = parity.run_oracle(wl, bufs.host_W, bufs.inputs)
    g = full_check(wl, bufs, ref)
    check_verify(bufs, g)


# a vocabulary of 4133 16-column tiles: the streaming head's 2048 waves take balanced
# runs of 2 or 3 tiles (32 or 48 columns)
RAGGED_VOCAB = 16 * 4133


@pytest.mark.parametrize("case,batch,vocab", [("all_equal", 1, 0), ("tied_block", 1, 0),
                                              ("all_equal", 4, 0), ("tied_block", 4, 0),
                                              ("all_equal", 1, RAGGED_VOCAB),
                                              ("tied_block", 1, RAGGED_VOCAB)])
def test_mid_step_head_run_selection_ties(case, batch, vocab):
    """The 1024-wide drafter takes the selection from the output head's column-run
    statistics: at batch 1 the streaming head's runs (one 16-column tile per wave at
    V = 8192; 2 or 3 tiles at the ragged vocabulary), at batch 4 the many-row head's
    256-column tiles.  Every head row equal: all logits tie, every run reaches the
    threshold and the exact scan must return ids 0..K-1 with log-prob -log(V).  A block
    of 40 equal rows among random ones (across run boundaries): candidates tie inside
    the run lists, and the top K must still be exact by (logit desc, id asc) on the
    GPU's own logits."""
    s = synth.MID if not vocab else dataclasses.replace(synth.MID, vocab=vocab)
    wl = dataclasses.replace(synth.WORKLOADS["tiny"], shape=s, batch=batch, ctx_len=96,
                             seed=141)
    say(f"[step] mid head-run selection, {case}, batch {batch}, vocab {s.vocab}")
    W = synth.make_weights(s, wl.seed)
    E = W["embed"].copy()
    if case == "all_equal":
        E[:] = E[:1]
    else:
        # 40 copies of proposal row 0's best head row: 41 equal top logits in that row
        probe = runner.StepBuffers(wl, weights=W)
        probe.step(dbg=False)
        u = int(probe.cand_ids.cpu().numpy()[0, 0, 0])
        E[1000:1040] = E[u]
        del probe
    W["embed"] = E
    W["lm_head"] = E
    bufs = runner.StepBuffers(wl, weights=W)
    bufs.step()
    g = gpu_outputs(bufs)
    K, V = s.top_k, s.vocab
    if case == "all_equal":
        assert (g["ids"] == np.arange(K)).all()
        assert np.allclose(g["lp"], -np.log(V), atol=1e-4)
    else:
        want = sorted([u] + list(range(1000, 1040)))[:K]
        assert g["ids"][0, 0].tolist() == want
    parity.check_topk_reanchored(g["logits"], g["ids"], g["lp"], K)
    ref = parity.run_oracle(wl, W, bufs.inputs)
    assert np.abs(g["logits"] - ref["logits"]).max() <= parity.LOGIT_MAX_ABS


def test_mid_step_ragged_head_runs():
    """Full parity at a vocabulary whose 16-column tiles do not divide evenly over the
    streaming head's waves (balanced runs of 2 or 3 tiles), with the selector's
    codebooks N(0, 1) so that the path depends on every candidate."""
    s = dataclasses.replace(synth.MID, vocab=RAGGED_VOCAB)
    wl = dataclasses.replace(synth.WORKLOADS["tiny"], shape=s, batch=1, ctx_len=96, seed=143)
    say(f"[step] mid ragged head runs, vocab {s.vocab}")
    W = synth.make_weights(s, wl.seed, code_std=1.0)
    bufs = runner.StepBuffers(wl, weights=W)
    bufs.step()
    torch.cuda.synchronize()
    ref = parity.run_oracle(wl, bufs.host_W, bufs.inputs)
    g = full_check(wl, bufs, ref)
    check_verify(bufs, g)
