"""The oracle's elementary operations against library routines and closed forms (CPU)."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import draft
from oracle.bf16 import bf16_to_f64, f64_to_bf16, round_bf16


def test_bf16_conversion_exact_and_nearest():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(10000) * 10.0 ** rng.integers(-5, 5, 10000)
    b = f64_to_bf16(x)
    tb = torch.from_numpy(x).to(torch.bfloat16)            # library RNE from float64
    assert np.array_equal(b, tb.view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(bf16_to_f64(b), tb.to(torch.float64).numpy())
    # exactly representable values survive
    assert np.array_equal(round_bf16(np.array([1.0, -2.5, 0.0078125])), [1.0, -2.5, 0.0078125])


def test_rmsnorm_matches_torch():
    rng = np.random.default_rng(1)
    v = rng.standard_normal((3, 5, 64))
    g = rng.standard_normal(64)
    ref = F.rms_norm(torch.from_numpy(v), (64,), torch.from_numpy(g), eps=1e-6).numpy()
    assert np.allclose(draft.rmsnorm(v, g, 1e-6), ref, rtol=1e-13, atol=1e-14)


def test_silu_softmax_logsumexp_match_torch():
    rng = np.random.default_rng(2)
    v = rng.standard_normal((4, 100)) * 5
    t = torch.from_numpy(v)
    assert np.allclose(draft.silu(v), F.silu(t).numpy(), rtol=1e-14, atol=1e-15)
    assert np.allclose(draft.softmax(v), torch.softmax(t, -1).numpy(), rtol=1e-13)
    assert np.allclose(draft.logsumexp(v), torch.logsumexp(t, -1).numpy(), rtol=1e-14)


def test_topk_matches_torch_and_tie_rule():
    rng = np.random.default_rng(3)
    v = rng.standard_normal(5000)
    idx = draft.topk_desc(v, 16)
    ref = torch.topk(torch.from_numpy(v), 16).indices.numpy()
    assert np.array_equal(idx, ref)
    # ties: equal values are ordered by lower index first
    w = np.zeros(10)
    w[[7, 2, 5]] = 1.0
    assert list(draft.topk_desc(w, 4)) == [2, 5, 7, 0]


def test_rope_is_rotation_with_relative_phase():
    rng = np.random.default_rng(4)
    d = 128
    x = rng.standard_normal((3, d))
    pos = np.array([0, 17, 262143])
    y = draft.rope(x, pos, 1e6)
    assert np.allclose(y[0], x[0])                                   # position 0 = identity
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1))
    # complex-number form: (x_i + i x_{i+d/2}) * exp(i p f_i)
    f = 1e6 ** (-np.arange(d // 2) * 2.0 / d)
    z = (x[:, :d // 2] + 1j * x[:, d // 2:]) * np.exp(1j * pos[:, None] * f[None, :])
    assert np.allclose(y, np.concatenate([z.real, z.imag], -1), atol=1e-9)
    # <rope(q, p1), rope(k, p2)> depends only on p1 - p2
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    a = draft.rope(np.stack([q]), [100], 1e6) @ draft.rope(np.stack([k]), [40], 1e6).T
    b = draft.rope(np.stack([q]), [1060], 1e6) @ draft.rope(np.stack([k]), [1000], 1e6).T
    assert np.allclose(a, b)


def test_attention_matches_sdpa_with_gqa():
    rng = np.random.default_rng(5)
    T, S, n_q, n_kv, d = 8, 40, 8, 2, 64
    q = rng.standard_normal((T, n_q, d))
    kb, vb = rng.standard_normal((T, n_kv, d)), rng.standard_normal((T, n_kv, d))
    kc, vc = rng.standard_normal((S, n_kv, d)), rng.standard_normal((S, n_kv, d))
    o = draft.attention(q, kb, vb, kc, vc, n_q, n_kv)
    K = torch.from_numpy(np.concatenate([kc, kb])).permute(1, 0, 2)       # [n_kv, S+T, d]
    Vv = torch.from_numpy(np.concatenate([vc, vb])).permute(1, 0, 2)
    K = K.repeat_interleave(n_q // n_kv, dim=0)
    Vv = Vv.repeat_interleave(n_q // n_kv, dim=0)
    ref = F.scaled_dot_product_attention(torch.from_numpy(q).permute(1, 0, 2), K, Vv)
    assert np.allclose(o, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_attention_equal_keys_average_values():
    rng = np.random.default_rng(6)
    T, S, n_q, n_kv, d = 4, 10, 2, 1, 16
    q = rng.standard_normal((T, n_q, d))
    k = np.ones((S + T, n_kv, d))
    v = rng.standard_normal((S + T, n_kv, d))
    o = draft.attention(q, k[S:], v[S:], k[:S], v[:S], n_q, n_kv)
    assert np.allclose(o, np.broadcast_to(v.mean(0)[:, None, :].repeat(n_q, 1)[0], o.shape))


def test_dynamic_conv_hand_example():
    """Two positions, one head of width 2.  W_c rows: a-row, b-row."""
    o = np.array([[[1.0, 2.0]], [[3.0, 4.0]]])              # [T=2, n_q=1, d=2]
    w = np.array([[1.0, 0.0], [0.0, 1.0]])                  # a = o[0], b = o[1] (per row)
    y = draft.dynamic_conv(o, w)
    # t=0: a=1, b=2, prev=0 -> y = 1*[1,2]            = [1, 2]
    # t=1: a=3, b=4, prev=[1,2] -> y = 3*[3,4]+4*[1,2] = [13, 20]
    assert np.array_equal(y, np.array([[[1.0, 2.0]], [[13.0, 20.0]]]))


def test_dynamic_conv_degenerate_taps():
    rng = np.random.default_rng(7)
    o = rng.standard_normal((8, 4, 16))
    assert np.array_equal(draft.dynamic_conv(o, np.zeros((8, 64))), np.zeros_like(o))
    # a = 1, b = 0 for every head -> y = o: give o a constant channel 0 equal to 1
    # and let row h of W_c read head h's channel 0
    o2 = o.copy()
    o2[:, :, 0] = 1.0
    w = np.zeros((8, 64))
    for h in range(4):
        w[h, h * 16] = 1.0
    y = draft.dynamic_conv(o2, w)
    assert np.allclose(y, o2)


@pytest.mark.parametrize("V,K", [(4096, 4), (50000, 16)])
def test_lm_head_topk_against_torch(V, K):
    rng = np.random.default_rng(8)
    H = 64
    E = f64_to_bf16(rng.standard_normal((V, H)) * 0.02)
    f = rng.standard_normal((2, 3, H))
    r = draft.lm_head_topk(f, E, K, chunk=1000)
    logits = torch.from_numpy(f) @ torch.from_numpy(bf16_to_f64(E)).T
    lse = torch.logsumexp(logits, -1)
    top = torch.topk(logits, K, dim=-1)
    assert np.array_equal(r["cand_ids"], top.indices.numpy())
    assert np.allclose(r["cand_logp"], (top.values - lse[..., None]).numpy(), rtol=1e-12)
    assert np.allclose(r["logits"], logits.numpy(), rtol=1e-12, atol=1e-12)
