"""dflash_draft_step_noalloc against dflash_draft_step (GPU).

The no-allocation step runs the same kernels on the library's static device scratch
instead of a caller workspace, so its results must equal those of the workspace entry
point bit for bit (the kernels are deterministic): the chosen path, candidates and
log-probabilities, the hidden states and logits, and the appended cache rows.  Two
calls in a row, the second with a smaller input (the scratch keeps the first call's
contents), then a configuration too large for the scratch is refused on the host.
"""
import ctypes
import dataclasses
import sys

import numpy as np
import pytest
import torch

from block_diffusion_draft_amd import binding, runner, synth

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def outputs(b):
    torch.cuda.synchronize()
    return dict(draft=b.draft.cpu(), ids=b.cand_ids.cpu(), lp=b.cand_logp.cpu(),
                hidden=b.dbg_hidden.cpu(), logits=b.dbg_logits.cpu(), k=b.k_cache.cpu(),
                v=b.v_cache.cpu())


def run_pair(wl, W=None, inputs=None):
    ref = runner.StepBuffers(wl, weights=W, inputs=inputs)
    ref.step()
    want = outputs(ref)
    noa = runner.StepBuffers(wl, weights=ref.host_W, inputs=ref.inputs)
    binding.draft_step_noalloc(noa.cfg, noa.dw, noa.taps, noa.last, noa.ctx_len, noa.k_cache,
                               noa.v_cache, noa.draft, noa.cand_ids, noa.cand_logp,
                               noa.dbg_hidden, noa.dbg_logits)
    got = outputs(noa)
    for k in want:
        assert torch.equal(want[k], got[k]), k
    return got


def test_noalloc_step_equals_workspace_step_twice():
    s = synth.MID
    big = dataclasses.replace(synth.WORKLOADS["tiny"], shape=s, batch=3, ctx_len=96, seed=71)
    need = binding.workspace_bytes(binding.make_config(s), big.batch, big.t_new)
    say(f"[noalloc] mid drafter, batch 3 (workspace {need / 2**20:.2f} MiB)")
    run_pair(big)
    small = dataclasses.replace(synth.WORKLOADS["tiny"], batch=1, seed=72)
    say("[noalloc] tiny drafter, batch 1, after the larger call")
    run_pair(small)


def test_noalloc_step_refuses_a_workspace_beyond_the_scratch():
    s = synth.FULL
    cfg = binding.make_config(s)
    assert binding.workspace_bytes(cfg, 16, 8) > binding.NOALLOC_SCRATCH_BYTES
    assert binding.workspace_bytes(cfg, 1, 8) <= binding.NOALLOC_SCRATCH_BYTES
    fake = 0x10000
    w = binding.Weights()
    for f in ("fc", "hidden_norm", "final_norm", "embed", "lm_head", "mask_emb", "sel_proj",
              "code_a", "code_b"):
        setattr(w, f, fake)
    for l in range(s.n_layers):
        for f, _ in binding.LayerWeights._fields_:
            setattr(w.layer[l], f, fake)
    w.linear_layout = binding.LAYOUT_TILED
    rc = binding.lib().dflash_draft_step_noalloc(ctypes.byref(cfg), ctypes.byref(w), 16, fake, 8,
                                                 fake, fake, fake, fake, 64, fake, fake, fake,
                                                 None, None, None)
    assert rc == -7
