"""A multi-step drafting loop on the GPU, checked step by step against the oracle.

The loop (FastFlowLM card "Qwen3.8-27B-DFlash2-NPU2", section "How it is used": the
draft proposes a block, the target checks all proposals in one pass, keeps the longest
agreeing prefix plus one token of its own; the draft then continues from there):

  draft step (t_new context rows appended) -> synthetic target's greedy tokens ->
  dflash_verify_prefix -> the k + 1 committed tokens become the next step's t_new = k + 1
  context rows (their taps), ctx_len grows by this step's t_new, the anchor becomes
  the last committed token -> next draft step.

With sampled acceptance (dflash_verify_sampled, temperature 1.0, top-k 20, top-p
0.95) the target's logits for the step are synthetic: N(0, 2) with the drafted token
lifted above its row's maximum at 9 of 10 positions.

The target is synthetic (seeded, no trained weights): the taps of a context row are
bf16 N(0, 1) drawn from the row's sequence and absolute position, and its greedy token
after block position j agrees with the drafted token with probability 3/4 (seeded),
so acceptance lengths vary from step to step.  The cache rows stay on the device from
step to step; each step is compared with the oracle run on the same state (the
caches read back from the device, the same taps, anchor and context length), to the
single-step bars; the drafted tokens equal the oracle's own path, which alone builds
the synthetic target and the expected acceptance outputs (compared exactly).
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

from block_diffusion_draft_amd import binding, runner, synth
from oracle import sample
from oracle import select as oselect
from oracle.bf16 import bf16_to_f64
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


def oracle_path(ref, W, s):
    """The oracle's drafted tokens: Viterbi over its own candidates."""
    ids, lp = ref["cand_ids"][0], ref["cand_logp"][0]
    T = oselect.pair_scores(ids, bf16_to_f64(W["code_a"]), bf16_to_f64(W["code_b"]),
                            s.pair_scale)
    path, _ = oselect.viterbi(lp, T)
    return ids[np.arange(ids.shape[0]), path].astype(np.int32)


def loop_taps(seed, b, pos, t_new, width):
    """Taps of the context rows at absolute positions pos .. pos + t_new - 1."""
    return np.stack([synth.normal_bf16(seed, f"loop.taps.{b}.{pos + i}", (width,), 1.0)
                     for i in range(t_new)])


@pytest.mark.parametrize("block,accept", [(8, "greedy"), (5, "greedy"), (8, "sampled")])
def test_greedy_loop_tiny(block, accept):
    shape = dataclasses.replace(synth.TINY, block=block)
    steps, seed, n0 = 6, 31 + block + (accept == "sampled"), 40
    wl0 = dataclasses.replace(synth.WORKLOADS["tiny"], shape=shape, seed=seed, ctx_len=n0,
                              t_new=8, cache_extra=steps * 8)
    say(f"[loop] tiny block {block}, {steps} steps, {accept} acceptance")
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
        path = oracle_path(ref, bufs.host_W, shape)
        assert np.array_equal(g["draft"][0], path)
        pos = ctx + t_new
        if accept == "greedy":
            y = target_greedy(seed, 0, pos, path, V)
            bufs.verify(torch.from_numpy(y[None]).cuda())
            ra, ro = verify_prefix(path[None], y[None])
        else:
            z = synth.target_logits(seed, f"loop.z.{pos}", path[None], V)
            u = synth.uniform(seed, f"loop.u.{pos}", (1, P + 1, 2))
            ws = torch.empty(binding.verify_sampled_workspace_bytes(1, P, V),
                             dtype=torch.uint8, device="cuda")
            binding.verify_sampled(bufs.draft, torch.from_numpy(z).cuda(),
                                   torch.from_numpy(u).cuda(), 1.0, 20, 0.95, ws,
                                   bufs.accept_len, bufs.out_tokens)
            ra, ro, mg = sample.verify_sampled(path[None], z.astype(np.float64), u, 1.0, 20,
                                               0.95)
            assert mg[0] > 1e-5          # every decision clear of fp32 rounding
        torch.cuda.synchronize()
        k = int(bufs.accept_len.cpu().numpy()[0])
        out = bufs.out_tokens.cpu().numpy()[0]
        assert k == int(ra[0]) and np.array_equal(out, ro[0])
        say(f"  step {step}: ctx {ctx}, t_new {t_new}, accepted {k} of {P}")
        lengths.append(k)
        # hand-off: this step's rows are cached; the k + 1 committed tokens are next
        ctx += t_new
        t_new = k + 1
        last = int(out[k])
        taps = loop_taps(seed, 0, ctx, t_new, width)[None]
    assert len(set(lengths)) > 1, lengths      # the acceptance length varied
