"""A multi-step greedy drafting loop on the GPU, checked step by step against the oracle.

The loop (FastFlowLM card "Qwen3.8-27B-DFlash2-NPU2", section "How it is used": the
draft proposes a block, the target checks all proposals in one pass, keeps the longest
agreeing prefix plus one token of its own; the draft then continues from there):

  draft step (t_new context rows appended) -> synthetic target's greedy tokens ->
  dflash_verify_prefix -> the k + 1 committed tokens become the next step's t_new = k + 1
  context rows (their taps), ctx_len grows by this step's t_new, the anchor becomes
  the last committed token -> next draft step.

The target is synthetic (seeded, no trained weights): the taps of a context row are
bf16 N(0, 1) drawn from the row's sequence and absolute position, and its greedy token
after block position j agrees with the drafted token with probability 3/4 (seeded),
so acceptance lengths vary from step to step.  The cache rows stay on the device from
step to step; each step is compared with the oracle run on the same state (the
caches read back from the device, the same taps, anchor and context length), to the
single-step bars, and the acceptance outputs exactly.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

from block_diffusion_draft_amd import binding, runner, synth
from oracle.verify import verify_prefix
from tests import parity
from tests.test_gpu_step import full_check, gpu_outputs

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def target_greedy(seed, b, pos, path, V):
    """Synthetic target: greedy token after block position j (j = 0..P) of the step whose
    block starts at absolute position `pos`.  Agrees with path[j] with probability 3/4."""
    P = len(path)
    u = synth.randint(seed, f"loop.accept.{b}.{pos}", (P + 1,), 0, 4)
    other = synth.randint(seed, f"loop.other.{b}.{pos}", (P + 1,), 0, V)
    y = other.astype(np.int32)
    for j in range(P):
        if u[j] != 0:
            y[j] = path[j]
        elif other[j] == path[j]:
            y[j] = (path[j] + 1) % V
    return y


def loop_taps(seed, b, pos, t_new, width):
    """Taps of the context rows at absolute positions pos .. pos + t_new - 1."""
    return np.stack([synth.normal_bf16(seed, f"loop.taps.{b}.{pos + i}", (width,), 1.0)
                     for i in range(t_new)])


@pytest.mark.parametrize("block", [8, 5])
def test_greedy_loop_tiny(block):
    shape = dataclasses.replace(synth.TINY, block=block)
    steps, seed, n0 = 6, 31 + block, 40
    wl0 = dataclasses.replace(synth.WORKLOADS["tiny"], shape=shape, seed=seed, ctx_len=n0,
                              t_new=8, cache_extra=steps * 8)
    say(f"[loop] tiny block {block}, {steps} steps")
    bufs = runner.StepBuffers(wl0, poison_outside_window=False)
    P, V = block - 1, shape.vocab
    width = shape.n_taps * shape.hidden
    # workspace for the largest t_new
    ctx, last, t_new = n0, int(bufs.inputs["last_token"][0]), 8
    taps = loop_taps(seed, 0, ctx, t_new, width)[None]
    lengths = []
    for step in range(steps):
        wl = dataclasses.replace(wl0, ctx_len=ctx, t_new=t_new)
        inputs = dict(taps=taps, last_token=np.array([last], dtype=np.int32),
                      ctx_len=np.array([ctx], dtype=np.int32),
                      k_cache=bufs.k_cache.cpu().numpy().view(np.uint16),
                      v_cache=bufs.v_cache.cpu().numpy().view(np.uint16))
        bufs.inputs = inputs
        bufs.wl = wl
        bufs.taps = torch.from_numpy(taps.view(np.int16)).cuda()
        bufs.last = torch.tensor([last], dtype=torch.int32, device="cuda")
        bufs.ctx_len = torch.tensor([ctx], dtype=torch.int32, device="cuda")
        bufs.step()
        ref = parity.run_oracle(wl, bufs.host_W, inputs)
        g = full_check(wl, bufs, ref)
        path = g["draft"][0]
        y = target_greedy(seed, 0, ctx + t_new, path, V)
        bufs.verify(torch.from_numpy(y[None]).cuda())
        torch.cuda.synchronize()
        k = int(bufs.accept_len.cpu().numpy()[0])
        out = bufs.out_tokens.cpu().numpy()[0]
        ra, ro = verify_prefix(g["draft"], y[None])
        assert k == int(ra[0]) and np.array_equal(out, ro[0])
        say(f"  step {step}: ctx {ctx}, t_new {t_new}, accepted {k} of {P}")
        lengths.append(k)
        # hand-off: this step's rows are cached; the k + 1 committed tokens are next
        ctx += t_new
        t_new = k + 1
        last = int(out[k])
        taps = loop_taps(seed, 0, ctx, t_new, width)[None]
    assert len(set(lengths)) > 1, lengths      # the acceptance length varied
