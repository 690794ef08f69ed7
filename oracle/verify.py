"""Greedy accept-longest-prefix (test infrastructure only).

Source: FastFlowLM card "Qwen3.8-27B-DFlash2-NPU2", section "How it is used":
the main model checks the 7 drafted tokens in one pass and keeps the longest
prefix it agrees with, plus one token of its own; section "FastFlowLM
measurements": drafted tokens are compared with the model's own most likely
token (the sampler is skipped).

target[i] is the target's greedy token after block position i (position 0 is
the last accepted token), so draft[j] is accepted while draft[j] == target[j].
"""
import numpy as np


def verify_prefix(draft, target):
    """draft int [B, n], target int [B, n+1] -> (accept_len [B], out [B, n+1]).

    accept_len = k = number of leading j with draft[j] == target[j] (0..n);
    out = draft[0..k-1], target[k], then -1 padding.
    """
    draft = np.asarray(draft)
    target = np.asarray(target)
    B, n = draft.shape
    assert target.shape == (B, n + 1)
    acc = np.zeros(B, dtype=np.int32)
    out = np.full((B, n + 1), -1, dtype=np.int32)
    for b in range(B):
        k = 0
        while k < n and draft[b, k] == target[b, k]:
            k += 1
        acc[b] = k
        out[b, :k] = draft[b, :k]
        out[b, k] = target[b, k]
    return acc, out
