"""GPU parity of the batched draft steps at the full 27B-draft shape.

* 16 sequences, Q4_K weights, 32768 cached rows each (window 2048);
* 64 sequences, bf16 weights, 8192 cached rows each.

The float64 oracle runs on a seeded sample of the sequences (sequences are
independent, so a sample is a complete check of those rows); on every sequence
the properties that hold at any size are checked: top-K ids and log-probs
re-anchored on the GPU's own logits, the path equal to the Viterbi path over the
GPU's own candidates, finite outputs, and the prefix acceptance.
"""
import gc
import sys

import numpy as np
import pytest
import torch

from block_diffusion_draft_amd import runner, synth
from tests import parity
from tests.test_gpu_step import check_verify, full_check, gpu_outputs

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def sample_sequences(wl, n=2):
    rng = np.random.default_rng(1000 + wl.seed)
    return sorted(rng.choice(wl.batch, size=n, replace=False).tolist())


def run_batched(key):
    wl = synth.WORKLOADS[key]
    say(f"[step] {wl.name}: generating inputs")
    bufs = runner.StepBuffers(wl)
    say("  running GPU step")
    bufs.step()
    torch.cuda.synchronize()
    g = gpu_outputs(bufs)
    assert np.isfinite(g["logits"]).all() and np.isfinite(g["hidden"]).all()
    say("  properties on every sequence")
    parity.check_topk_reanchored(g["logits"], g["ids"], g["lp"], wl.shape.top_k)
    W = bufs.host_W
    ties = parity.check_paths(g["ids"], g["lp"], g["draft"], W["code_a"], W["code_b"],
                              wl.shape.pair_scale)
    check_verify(bufs, g)
    seqs = sample_sequences(wl)
    say(f"  running oracle on sequences {seqs} (path near-ties over the batch: {ties})")
    ref = parity.run_oracle(wl, W, bufs.inputs, seqs=seqs)
    full_check(wl, bufs, ref, seqs=seqs)
    del bufs
    gc.collect()
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_full_step_b16_q4k_parity():
    run_batched("full_b16")


@pytest.mark.timeout(900)
def test_full_step_b64_bf16_parity():
    run_batched("full_b64_bf16")
