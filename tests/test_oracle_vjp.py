"""Pins for the fp64 gradient oracle (oracle/attention_vjp.py).

Each check ties it to something other than itself: reverse-mode autodiff of a
dense masked attention and of PyTorch's scaled_dot_product_attention, the
adjoint identity with the forward-mode JVP oracle (itself pinned in
test_oracle.py), central finite differences of the JVP oracle's primal, and
the sum rules that follow from the softmax (shifting every key by one vector
changes nothing; the attention weights of a row sum to one).
"""
import math

import numpy as np
import pytest
import torch

from oracle import MaskLayout, RectMask, attn_jvp_ref, attn_vjp_ref, attn_vjp_sampled, dense_mask, key_ranges

LAYOUTS = [
    MaskLayout("full", 3, 4),
    MaskLayout("block_causal", 5, 4, 1),
    MaskLayout("block_causal", 5, 3, 2),
    MaskLayout("tf_clean_noisy", 3, 4, 1),
    MaskLayout("tf_clean_noisy", 4, 2, 2),
    RectMask(14, ((0, 5, 0, 5), (5, 14, 0, 3), (5, 14, 8, 14), (9, 12, 4, 6))),
]
IDS = ["full", "frame_causal", "chunk2_ragged", "tf", "tf_chunk2", "rects"]


def _rand(L, d=8, B=1, H=2, seed=0, n=4):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((B, H, L, d)) for _ in range(n)]


def _dense_grads(q, k, v, do, mask, c):
    """Reverse-mode autodiff of <dO, softmax(c q k^T + M) v> in float64."""
    dm = torch.from_numpy(dense_mask(mask))
    qt, kt, vt = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    s = (qt @ kt.transpose(-1, -2)) * c
    s = s.masked_fill(~dm, float("-inf"))
    p = torch.softmax(s, dim=-1)
    p = torch.nan_to_num(p)  # rows with no allowed key: zero output
    o = p @ vt
    (o * torch.from_numpy(do)).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


@pytest.mark.parametrize("mask", LAYOUTS, ids=IDS)
def test_matches_reverse_mode_autodiff(mask):
    q, k, v, do = _rand(mask.seq_len, seed=1)
    c = 0.41
    got = attn_vjp_ref(q, k, v, do, mask, scale=c)
    want = _dense_grads(q, k, v, do, mask, c)
    for g, w in zip(got, want):
        np.testing.assert_allclose(g, w, rtol=1e-10, atol=1e-12)


def test_full_and_causal_special_cases_match_sdpa_backward():
    for mask, causal in ((MaskLayout("full", 2, 9), False), (MaskLayout("block_causal", 17, 1, 1), True)):
        q, k, v, do = _rand(mask.seq_len, d=16, seed=2)
        qt, kt, vt = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal)
        (o * torch.from_numpy(do)).sum().backward()
        got = attn_vjp_ref(q, k, v, do, mask)
        for g, w in zip(got, (qt.grad, kt.grad, vt.grad)):
            np.testing.assert_allclose(g, w.numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("mask", LAYOUTS, ids=IDS)
def test_adjoint_identity_with_the_jvp_oracle(mask):
    # <dO, J t> = <J^T dO, t> for every tangent t and cotangent dO
    q, k, v, do = _rand(mask.seq_len, seed=3)
    tq, tk, tv = _rand(mask.seq_len, seed=4, n=3)
    c = 0.29
    _, to, _ = attn_jvp_ref(q, k, v, tq, tk, tv, mask, scale=c)
    dq, dk, dv = attn_vjp_ref(q, k, v, do, mask, scale=c)
    lhs = float((do * to).sum())
    rhs = float((dq * tq).sum() + (dk * tk).sum() + (dv * tv).sum())
    assert abs(lhs - rhs) <= 1e-11 * max(1.0, abs(lhs))


@pytest.mark.parametrize("mask", LAYOUTS[:4], ids=IDS[:4])
def test_matches_central_finite_differences(mask):
    q, k, v, do = _rand(mask.seq_len, seed=5)
    c = 0.5
    dq, dk, dv = attn_vjp_ref(q, k, v, do, mask, scale=c)
    rng = np.random.default_rng(6)
    f = lambda q_, k_, v_: float((do * attn_jvp_ref(q_, k_, v_, q_, k_, v_, mask, scale=c)[0]).sum())
    eps = 1e-6
    for _ in range(3):
        eq, ek, ev = (rng.standard_normal(q.shape) for _ in range(3))
        fd = (f(q + eps * eq, k + eps * ek, v + eps * ev) - f(q - eps * eq, k - eps * ek, v - eps * ev)) / (2 * eps)
        an = float((dq * eq).sum() + (dk * ek).sum() + (dv * ev).sum())
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an))


@pytest.mark.parametrize("mask", LAYOUTS, ids=IDS)
def test_sum_rules(mask):
    q, k, v, do = _rand(mask.seq_len, seed=7)
    dq, dk, dv = attn_vjp_ref(q, k, v, do, mask)
    # shifting every key by one vector leaves the output unchanged: sum_j dk_j = 0
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    # the weights of a row sum to one: sum_j dv_j = sum of dO over rows that see keys
    seen = np.array([len(key_ranges(mask, i)) > 0 for i in range(mask.seq_len)])
    np.testing.assert_allclose(dv.sum(axis=2), do[:, :, seen].sum(axis=2), atol=1e-12)
    # masked-out structure: no gradient for rows without keys / keys nobody sees
    dm = dense_mask(mask)
    assert not dq[:, :, ~dm.any(axis=1)].any()
    assert not dk[:, :, ~dm.any(axis=0)].any() and not dv[:, :, ~dm.any(axis=0)].any()


def test_rows_and_keys_nobody_uses():
    mask = RectMask(12, ((0, 4, 0, 4), (8, 12, 0, 6)))  # rows 4..7 see nothing; keys 6..11 unseen
    q, k, v, do = _rand(12, seed=8)
    dq, dk, dv = attn_vjp_ref(q, k, v, do, mask)
    assert not dq[:, :, 4:8].any() and not dk[:, :, 6:].any() and not dv[:, :, 6:].any()
    want = _dense_grads(q, k, v, do, mask, 1 / math.sqrt(8))
    for g, w in zip((dq, dk, dv), want):
        np.testing.assert_allclose(g, w, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("mask", LAYOUTS, ids=IDS)
def test_sampled_rows_and_keys_match_the_full_evaluation(mask):
    q, k, v, do = _rand(mask.seq_len, B=2, H=2, seed=9)
    dq, dk, dv = attn_vjp_ref(q, k, v, do, mask)
    L = mask.seq_len
    rows, keys = [0, L - 1, L // 2, 3, 3], [L - 1, 0, L // 3, 5]
    heads = [(0, 1), (1, 0)]
    sq, sk, sv = attn_vjp_sampled(q, k, v, do, mask, rows, keys, heads)
    for bh in heads:
        np.testing.assert_allclose(sq[bh], dq[bh][rows], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(sk[bh], dk[bh][keys], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(sv[bh], dv[bh][keys], rtol=1e-12, atol=1e-13)
