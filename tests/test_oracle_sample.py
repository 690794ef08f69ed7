"""Pins of the sampled-acceptance oracle (exact rejection sampling of a drafted block).

Mindket kit page "Qwen3.8-27B-DFlash2-GGUF by z-lab", "For newcomers and experts": with
sampling the output keeps the target's distribution; "Good to know": the sampler is
temperature 1.0, top-p 0.95, top-k 20.  The pins: hand-computed truncated
distributions, the untruncated case against scipy's softmax, the top_k = 1 case against
greedy prefix acceptance, and Monte Carlo runs showing that every emitted token has the
target's distribution given the tokens before it (with a planted mistake in the
procedure, the same statistic rejects).
"""
import numpy as np
import pytest
from scipy.special import softmax
from scipy.stats import chisquare

from block_diffusion_draft_amd import synth
from oracle import sample
from oracle.verify import verify_prefix

P4 = np.array([0.5, 0.3, 0.15, 0.05])


def dist(logits, T=1.0, k=None, p=1.0):
    ids, probs, _ = sample.target_dist(np.asarray(logits, dtype=np.float64), T,
                                       k or len(logits), p)
    return list(ids), probs


@pytest.mark.parametrize("k,p,want_ids,want", [
    (4, 1.0, [0, 1, 2, 3], P4),
    (4, 0.9, [0, 1, 2], P4[:3] / 0.95),
    (4, 0.6, [0, 1], [0.625, 0.375]),
    (4, 0.45, [0], [1.0]),
    (2, 1.0, [0, 1], [0.625, 0.375]),
    (3, 0.7, [0, 1], [0.625, 0.375]),
])
def test_truncated_distributions_by_hand(k, p, want_ids, want):
    ids, probs = dist(np.log(P4), k=k, p=p)
    assert ids == want_ids
    np.testing.assert_allclose(probs, want, rtol=1e-12)


def test_temperature_and_id_mapping():
    # logits placed at ids 3, 0, 2, 1; temperature 2 takes square roots of the masses
    z = np.empty(4)
    z[[3, 0, 2, 1]] = np.log(P4)
    ids, probs = dist(z, T=2.0)
    assert ids == [3, 0, 2, 1]
    r = np.sqrt(P4)
    np.testing.assert_allclose(probs, r / r.sum(), rtol=1e-12)


def test_ties_take_the_lowest_id():
    ids, probs = dist([1.0, 2.0, 2.0, 0.0])
    assert ids == [1, 2, 0, 3]
    ids, _ = dist([2.0, 1.0, 1.0, 1.0], k=2)
    assert ids == [0, 1]


def test_untruncated_matches_scipy_softmax():
    z = synth.normal_f32(3, "sample.softmax", (300,), 2.0).astype(np.float64)
    ids, probs = dist(z, T=0.7)
    ref = softmax(z / 0.7)
    assert ids == list(np.lexsort((np.arange(300), -z)))
    np.testing.assert_allclose(probs, ref[ids], rtol=1e-10)


def test_draw_inverse_cdf():
    w = [0.25, 0.5, 0.25]
    assert [sample.draw(w, u)[0] for u in (0.0, 0.2499, 0.25, 0.7499, 0.75, 0.9999)] == \
        [0, 0, 1, 1, 2, 2]
    assert sample.draw(w, 0.25)[1] == 0.0              # on a boundary: no margin
    assert sample.draw([2.0, 6.0], 0.5)[0] == 1        # unnormalised weights


def test_top_k_one_is_greedy_prefix_acceptance():
    B, n, V = 6, 7, 50
    z = synth.normal_f32(4, "sample.greedy.z", (B, n + 1, V), 1.0)
    z[:, :, 7] = z.max(axis=2)          # ties at the maximum with a higher id
    z[:, :, 9] = z[:, :, 7]
    arg = np.argmax(z, axis=2)          # first maximum = lowest id
    draft = synth.randint(4, "sample.greedy.d", (B, n), 0, V)
    for b in range(B):
        draft[b, :b + 1] = arg[b, :b + 1]
    u = synth.uniform(4, "sample.greedy.u", (B, n + 1, 2))
    acc, out, _ = sample.verify_sampled(draft, z, u, 1.0, 1, 0.95)
    ra, ro = verify_prefix(draft, arg)
    assert list(acc) == list(ra)
    assert np.array_equal(out, ro)


def test_support_of_one_accepts_and_outside_support_rejects():
    z = np.log(np.array([[P4, P4, P4]]))           # [1, 3, 4]
    u = np.full((1, 3, 2), 0.999)
    # top_p 0.45 keeps token 0 only: drafting 0 is accepted whatever u is
    acc, out, _ = sample.verify_sampled([[0, 0]], z, u, 1.0, 4, 0.45)
    assert acc[0] == 2 and list(out[0]) == [0, 0, 0]
    # token 3 is outside the top-p 0.9 set: rejected even at u = 0
    acc, out, _ = sample.verify_sampled([[3, 0]], z, np.zeros((1, 3, 2)), 1.0, 4, 0.9)
    assert acc[0] == 0 and out[0, 0] == 0 and list(out[0, 1:]) == [-1, -1]


def test_margin_reports_a_decision_on_its_threshold():
    z = np.log(np.array([[[0.5, 0.5], [0.5, 0.5]]]))
    u = np.array([[[0.5, 0.1], [0.3, 0.3]]])
    acc, _, mg = sample.verify_sampled([[0]], z, u, 1.0, 2, 1.0)
    assert acc[0] == 0 and mg[0] == 0.0
    acc, _, mg = sample.verify_sampled([[0]], z, u - 0.2, 1.0, 2, 1.0)
    assert acc[0] == 1 and mg[0] > 0.09


# ---------------------------------------------------------------- exactness (Monte Carlo)

ROWS = np.log(np.array([[0.30, 0.25, 0.20, 0.15, 0.06, 0.04],
                        [0.05, 0.45, 0.22, 0.13, 0.10, 0.05],
                        [0.40, 0.10, 0.10, 0.25, 0.10, 0.05]]))
DRAFT = [2, 5]          # position 1's proposal lies outside its top-4 / top-p set
N_MC = 30000


def first_emitted_wrong(dists, u):
    """Position 0 of the procedure with a planted mistake: the residual keeps the
    rejected proposal."""
    ids, probs = dists[0]
    hit = np.nonzero(ids == DRAFT[0])[0]
    if len(hit) and u[0, 0] < probs[hit[0]]:
        return DRAFT[0]
    return ids[sample.draw(probs, u[0, 1])[0]]


def chi2_p(tokens, ids, probs):
    counts = np.array([np.sum(np.asarray(tokens) == t) for t in ids])
    assert counts.sum() == len(tokens)          # nothing outside the support
    return chisquare(counts, probs * len(tokens)).pvalue


@pytest.mark.parametrize("draft", [DRAFT, [0, 1]])
def test_emitted_tokens_follow_the_target_distribution(draft):
    dists = [sample.target_dist(r, 1.0, 4, 0.9)[:2] for r in ROWS]
    u = synth.uniform(8, "sample.mc.u", (N_MC, 3, 2)).astype(np.float64)
    outs = np.array([sample.accept_sequence(np.array(draft), dists, u[i])[1]
                     for i in range(N_MC)])
    sel = np.ones(N_MC, dtype=bool)
    for j in range(3):
        # given draft[:j] was emitted, the token emitted at j has distribution p_j
        assert chi2_p(outs[sel, j], *dists[j]) > 1e-4, j
        if j < 2:
            ids, probs = dists[j]
            p_x = probs[list(ids).index(draft[j])] if draft[j] in ids else 0.0
            nxt = sel & (outs[:, j] == draft[j])
            assert abs(nxt.sum() / sel.sum() - p_x) < 0.02
            assert (outs[sel & ~nxt, j + 1] == -1).all()
            sel = nxt
            if not sel.any():
                break
    assert (draft == DRAFT) == (not sel.any())   # draft[1] = 5 lies outside p_1's set


def test_planted_mistake_is_detected():
    dists = [sample.target_dist(r, 1.0, 4, 0.9)[:2] for r in ROWS]
    u = synth.uniform(8, "sample.mc.u", (N_MC, 3, 2)).astype(np.float64)
    outs = [first_emitted_wrong(dists, u[i]) for i in range(N_MC)]
    assert chi2_p(outs, *dists[0]) < 1e-6
