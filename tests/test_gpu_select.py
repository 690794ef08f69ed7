"""GPU selector paths where the transitions decide (through dflash_draft_step).

The candidate selector picks one consistent path through the top-K candidates of
the proposal positions (FastFlowLM card "Qwen3.8-27B-DFlash2-NPU2", spec table
"Draft" row: selector over the top 16 with rank-256 codebooks; Mindket kit page,
"For newcomers and experts").  With the workloads' N(0, 0.02) codebooks the pair
term is ~4e-4 and the path is almost always the per-position argmax; here the
codebooks are N(0, 1), so s <A[u], B[v]> ~ N(0, 1) outweighs the log-prob gaps.
The path must equal the float64 brute force over every path of the GPU's own
candidates (K = 4: 4^7 paths) or the Viterbi path (K = 16), and must differ from
the per-position argmax on most sequences, so a selector that dropped, transposed
or swapped the pair scores would fail.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

from block_diffusion_draft_amd import runner, synth
from oracle import select as oselect
from oracle.bf16 import bf16_to_f64
from tests import parity

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def path_checks(ids, lp, draft, code_a, code_b, s, brute):
    """Per sequence: the GPU path against the float64 optimum over its candidates
    (brute force or Viterbi; a different path only within PATH_MARGIN of the best
    score).  Returns the number of sequences whose path is not the argmax path."""
    A, Bm = bf16_to_f64(code_a), bf16_to_f64(code_b)
    not_argmax = 0
    for b in range(ids.shape[0]):
        T = oselect.pair_scores(ids[b], A, Bm, s)
        lp64 = lp[b].astype(np.float64)
        if brute:
            best, best_score, second = oselect.brute_force(lp64, T)
        else:
            best, best_score = oselect.viterbi(lp64, T)
        gp = np.array([list(ids[b, t]).index(draft[b, t]) for t in range(ids.shape[1])])
        if not np.array_equal(gp, best):
            m = best_score - oselect.path_score(lp64, T, gp)
            assert m < parity.PATH_MARGIN, (b, m, gp, best)
        not_argmax += bool(np.any(best != 0))
    return not_argmax


def test_tiny_selector_transitions_decide_k4():
    shape = synth.TINY
    total = nonarg = 0
    for seed in range(6):
        wl = dataclasses.replace(synth.WORKLOADS["tiny"], batch=4, seed=100 + seed)
        say(f"[select] tiny K=4 seed {wl.seed}, codebooks N(0, 1)")
        W = synth.make_weights(shape, wl.seed, code_std=1.0)
        bufs = runner.StepBuffers(wl, weights=W)
        bufs.step(dbg=False)
        torch.cuda.synchronize()
        ids, lp = bufs.cand_ids.cpu().numpy(), bufs.cand_logp.cpu().numpy()
        draft = bufs.draft.cpu().numpy()
        parity.check_paths(ids, lp, draft, W["code_a"], W["code_b"], shape.pair_scale)
        nonarg += path_checks(ids, lp, draft, W["code_a"], W["code_b"], shape.pair_scale,
                              brute=True)
        total += wl.batch
    say(f"  paths off the per-position argmax: {nonarg} of {total}")
    assert nonarg >= 0.75 * total


def test_mid_selector_transitions_decide_k16():
    """K = 16 candidates, rank 64, 8192-token vocabulary, 3 sequences."""
    shape = synth.MID
    wl = dataclasses.replace(synth.WORKLOADS["tiny"], shape=shape, batch=3, ctx_len=96,
                             seed=131)
    say("[select] mid K=16, codebooks N(0, 1)")
    W = synth.make_weights(shape, wl.seed, code_std=1.0)
    bufs = runner.StepBuffers(wl, weights=W)
    bufs.step(dbg=False)
    torch.cuda.synchronize()
    ids, lp = bufs.cand_ids.cpu().numpy(), bufs.cand_logp.cpu().numpy()
    draft = bufs.draft.cpu().numpy()
    nonarg = path_checks(ids, lp, draft, W["code_a"], W["code_b"], shape.pair_scale,
                         brute=False)
    say(f"  paths off the per-position argmax: {nonarg} of {wl.batch}")
    assert nonarg == wl.batch
