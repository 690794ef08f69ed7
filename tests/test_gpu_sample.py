"""GPU parity of sampled acceptance (dflash_verify_sampled) against the oracle.

Mindket kit page "Qwen3.8-27B-DFlash2-GGUF by z-lab", "For newcomers and experts" and
"Good to know": exact rejection sampling against the target's temperature / top-k /
top-p distribution.  Inputs are seeded: drafted tokens uniform over the vocabulary,
target logits N(0, 2) with the drafted token lifted 2 to 7 above its row's maximum at 9
of 10 positions (accepted lengths spread over 0 .. n), uniforms on [0, 1).

The bar: accepted lengths and emitted tokens equal the oracle's wherever every decision
the oracle took is more than MARGIN (relative to the mass involved) from its threshold;
the kernel decides in fp32, the oracle in float64, so a decision closer than that may
go either way.  For those rows the result must still be valid: the accepted tokens are
the drafted prefix, the emitted token lies in the target's truncated support, the rest
is -1.  At most a few rows per case may be that close.
"""
import sys

import numpy as np
import pytest
import torch

from block_diffusion_draft_amd import binding, synth
from oracle import sample

pytestmark = pytest.mark.gpu

MARGIN = 1e-5


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu(draft, z, u, T, k, p):
    B, n = draft.shape
    V = z.shape[2]
    ws = torch.empty(binding.verify_sampled_workspace_bytes(B, n, V), dtype=torch.uint8,
                     device="cuda")
    acc = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    out = torch.full((B, n + 1), -7, dtype=torch.int32, device="cuda")
    binding.verify_sampled(torch.from_numpy(np.ascontiguousarray(draft, dtype=np.int32)).cuda(),
                           torch.from_numpy(np.ascontiguousarray(z, dtype=np.float32)).cuda(),
                           torch.from_numpy(np.ascontiguousarray(u, dtype=np.float32)).cuda(),
                           T, k, p, ws, acc, out)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), out.cpu().numpy()


def check(draft, z, u, T, k, p, max_close=2):
    acc, out = run_gpu(draft, z, u, T, k, p)
    ra, ro, mg = sample.verify_sampled(draft, z.astype(np.float64), u, T, k, p)
    n = draft.shape[1]
    close = 0
    for b in range(draft.shape[0]):
        if mg[b] > MARGIN:
            assert acc[b] == ra[b] and np.array_equal(out[b], ro[b]), \
                (b, acc[b], ra[b], out[b], ro[b], mg[b])
            continue
        close += 1
        kb = int(acc[b])
        assert 0 <= kb <= n
        assert np.array_equal(out[b, :kb], draft[b, :kb])
        ids, _, _ = sample.target_dist(z[b, kb].astype(np.float64), T, k, p)
        assert out[b, kb] in ids
        assert (out[b, kb + 1:] == -1).all()
    assert close <= max_close, close
    return acc, out


def inputs(seed, B, n, V, lift=0.9, std=2.0):
    draft = synth.randint(seed, "sample.draft", (B, n), 0, V)
    z = synth.target_logits(seed, "sample.z", draft, V, std=std, lift=lift)
    u = synth.uniform(seed, "sample.u", (B, n + 1, 2))
    return draft, z, u


@pytest.mark.parametrize("T,k,p", [(1.0, 20, 0.95), (0.7, 5, 0.8), (1.3, 64, 1.0),
                                   (1.0, 1, 0.95), (1.0, 20, 0.01)])
def test_sampled_tiny_vocab_settings(T, k, p):
    say(f"[sampled] V 4096, B 64, n 7, T {T} top_k {k} top_p {p}")
    draft, z, u = inputs(20, 64, 7, 4096)
    acc, out = check(draft, z, u, T, k, p)
    if k > 1 and p > 0.5:
        assert len(set(acc.tolist())) >= 4           # acceptance lengths spread
    if k == 1 or p == 0.01:
        # a one-token support: the emitted token is the row's arg-max (lowest id on ties)
        for b in range(64):
            kb = acc[b]
            assert out[b, kb] == int(np.argmax(z[b, kb]))


@pytest.mark.parametrize("V,n", [(3001, 7), (50, 4), (5000, 1), (4096, 15), (1024, 63)])
def test_sampled_shapes(V, n):
    """Ragged vocabulary, vocabulary below one wave, fewer chunks than top_k (every logit
    is a candidate: the exact-scan path), more rows than waves, the largest n."""
    say(f"[sampled] V {V}, n {n}")
    draft, z, u = inputs(21 + n, 8, n, V)
    check(draft, z, u, 1.0, 20, 0.95)


@pytest.mark.parametrize("V,step", [(4096, 0.5), (248320, 4.0), (248320, 8.0)])
def test_sampled_ties_and_out_of_range_drafts(V, step):
    """Logits rounded to multiples of `step`: many exact ties at the top (at step 4 a few
    hundred logits reach the threshold, at step 8 thousands: more than the candidate
    list holds, so rows are scanned whole).  Drafted ids outside the vocabulary have
    probability 0 and are always rejected."""
    say(f"[sampled] ties V {V} step {step}, out-of-range drafts")
    B, n = 8, 7
    draft, z, u = inputs(23, B, n, V)
    z = np.round(z / step) * step
    draft[:2, 0] = -1
    draft[2:4, 0] = V + 5
    acc, out = check(draft, z, u, 1.0, 20, 0.93)
    assert (acc[:4] == 0).all()


def test_sampled_deterministic():
    draft, z, u = inputs(24, 16, 7, 4096)
    a1, o1 = run_gpu(draft, z, u, 1.0, 20, 0.95)
    a2, o2 = run_gpu(draft, z, u, 1.0, 20, 0.95)
    assert np.array_equal(a1, a2) and np.array_equal(o1, o2)


@pytest.mark.parametrize("B", [1, 16])
def test_sampled_full_vocab(B):
    """The 248320-token vocabulary of the 27B target, the pages' sampler settings."""
    say(f"[sampled] V 248320, B {B}, n 7")
    draft, z, u = inputs(30 + B, B, 7, 248320)
    check(draft, z, u, 1.0, 20, 0.95)
