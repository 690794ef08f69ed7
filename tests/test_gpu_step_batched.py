"""GPU parity of the batched draft steps at the full 27B-draft shape.

* 16 sequences, Q4_K weights, 32768 cached rows each (window 2048);
* 64 sequences, bf16 weights, 8192 cached rows each.

The float64 oracle runs on every sequence of the batch (one call, weights decoded
once), and each sequence is held to the bars of the single-sequence step: hidden
states per layer, logits, top-K validity, paths and the appended cache rows.  The
properties that hold at any size are checked as well: top-K ids and log-probs
re-anchored on the GPU's own logits, finite outputs, and the prefix acceptance.
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
    say(f"  running oracle on all {wl.batch} sequences (path near-ties: {ties})")
    ref = parity.run_oracle_chunked(wl, W, bufs.inputs, say=say)
    full_check(wl, bufs, ref)
    dl = np.abs(g["logits"] - ref["logits"]).max(axis=(1, 2))
    hid = [max(parity.rel_l2(g["hidden"][l, b], ref["hidden"][l, b])
               for l in range(ref["hidden"].shape[0])) for b in range(wl.batch)]
    say(f"  per sequence: logits max-abs worst {dl.max():.3e} (seq {int(dl.argmax())}), "
        f"median {np.median(dl):.3e}; hidden rel L2 worst {max(hid):.3e}")
    del bufs
    gc.collect()
    torch.cuda.empty_cache()


@pytest.mark.timeout(1100)
def test_full_step_b16_q4k_parity():
    run_batched("full_b16")


@pytest.mark.timeout(1100)
def test_full_step_b64_bf16_parity():
    run_batched("full_b64_bf16")
