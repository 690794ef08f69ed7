"""Pins of the greedy accept-longest-prefix oracle.

FastFlowLM card "Qwen3.8-27B-DFlash2-NPU2", section "How it is used": the main
model keeps the longest drafted prefix it agrees with plus one token of its own;
"Measured draft quality": kept-of-7 counts exclude that added token.
"""
import numpy as np

from oracle.verify import verify_prefix


def test_every_prefix_length():
    rng = np.random.default_rng(0)
    draft = rng.integers(0, 1000, size=(1, 7))
    for k in range(8):
        tgt = rng.integers(0, 1000, size=(1, 8))
        tgt[0, :k] = draft[0, :k]
        if k < 7:
            tgt[0, k] = (draft[0, k] + 1) % 1000
        acc, out = verify_prefix(draft, tgt)
        assert acc[0] == k
        assert list(out[0, :k]) == list(draft[0, :k])
        assert out[0, k] == tgt[0, k]
        assert (out[0, k + 1:] == -1).all()
        # tokens committed = kept + 1
        assert (out[0] >= 0).sum() == k + 1


def test_later_agreement_does_not_count():
    draft = np.array([[5, 6, 7, 8, 9, 10, 11]])
    tgt = np.array([[5, 0, 7, 8, 9, 10, 11, 12]])
    acc, out = verify_prefix(draft, tgt)
    assert acc[0] == 1 and list(out[0]) == [5, 0, -1, -1, -1, -1, -1, -1]


def test_batch_rows_independent():
    draft = np.array([[1, 2, 3, 4, 5, 6, 7]] * 3)
    tgt = np.array([[1, 2, 3, 4, 5, 6, 7, 99], [0] * 8, [1, 2, 9, 9, 9, 9, 9, 9]])
    acc, out = verify_prefix(draft, tgt)
    assert list(acc) == [7, 0, 2]
    assert list(out[0]) == [1, 2, 3, 4, 5, 6, 7, 99]
