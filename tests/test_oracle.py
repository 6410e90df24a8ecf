"""Pins for the fp64 oracle (oracle/attention_jvp.py).

Each check ties the oracle to something other than itself: finite differences
of its own primal, forward-mode autodiff of a dense masked attention, library
routines (scaled_dot_product_attention, logsumexp), per-element brute force, or
an invariant fixed by the mathematics of the JVP.
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle import MaskLayout, RectMask, attn_jvp_ref, dense_mask, key_ranges, allowed

LAYOUTS = [
    MaskLayout("full", 3, 4),
    MaskLayout("block_causal", 5, 4, 1),
    MaskLayout("block_causal", 5, 3, 2),
    MaskLayout("tf_clean_noisy", 3, 4, 1),
    MaskLayout("tf_clean_noisy", 4, 2, 2),
    RectMask(14, ((0, 5, 0, 5), (5, 14, 0, 3), (5, 14, 8, 14), (9, 12, 4, 6))),
]
IDS = ["full", "frame_causal", "chunk2_ragged", "tf", "tf_chunk2", "rects"]


def _rand(L, d=8, B=1, H=2, seed=0, sig=1.0):
    rng = np.random.default_rng(seed)
    return [sig * rng.standard_normal((B, H, L, d)) for _ in range(6)]


def _sdpa(q, k, v, mask, scale):
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(a)) for a in (q, k, v))
    dm = torch.from_numpy(dense_mask(mask))
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=dm, scale=scale).numpy()


@pytest.mark.parametrize("mask", LAYOUTS, ids=IDS)
def test_tangent_matches_central_finite_differences(mask):
    q, k, v, tq, tk, tv = _rand(mask.seq_len, seed=1)
    c = 0.37
    o, to, lse = attn_jvp_ref(q, k, v, tq, tk, tv, mask, scale=c)
    eps = 1e-6
    op, _, _ = attn_jvp_ref(q + eps * tq, k + eps * tk, v + eps * tv, tq, tk, tv, mask, scale=c)
    om, _, _ = attn_jvp_ref(q - eps * tq, k - eps * tk, v - eps * tv, tq, tk, tv, mask, scale=c)
    fd = (op - om) / (2 * eps)
    assert np.abs(to - fd).max() <= 1e-7 * max(1.0, np.abs(fd).max())


@pytest.mark.parametrize("mask", LAYOUTS, ids=IDS)
def test_tangent_matches_forward_mode_autodiff(mask):
    q, k, v, tq, tk, tv = _rand(mask.seq_len, seed=2)
    c = 1 / math.sqrt(8)
    dm = torch.from_numpy(dense_mask(mask))

    def attn(q_, k_, v_):
        s = (q_ @ k_.transpose(-1, -2)) * c
        s = s.masked_fill(~dm, float("-inf"))
        return torch.softmax(s, dim=-1) @ v_

    T = [torch.from_numpy(a) for a in (q, k, v, tq, tk, tv)]
    o_ad, to_ad = torch.func.jvp(attn, tuple(T[:3]), tuple(T[3:]))
    o, to, _ = attn_jvp_ref(q, k, v, tq, tk, tv, mask, scale=c)
    np.testing.assert_allclose(o, o_ad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(to, to_ad.numpy(), rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("mask", LAYOUTS, ids=IDS)
def test_primal_matches_sdpa_and_lse_matches_logsumexp(mask):
    q, k, v, tq, tk, tv = _rand(mask.seq_len, seed=3, sig=2.0)
    c = 0.25
    o, _, lse = attn_jvp_ref(q, k, v, tq, tk, tv, mask, scale=c)
    np.testing.assert_allclose(o, _sdpa(q, k, v, mask, c), rtol=1e-12, atol=1e-12)
    dm = dense_mask(mask)
    s = c * np.einsum("bhid,bhjd->bhij", q, k)
    ref = logsumexp(np.where(dm, s, -np.inf), axis=-1)
    np.testing.assert_allclose(lse, ref, rtol=1e-13, atol=1e-13)


def test_token_causal_special_case_matches_is_causal_sdpa():
    m = MaskLayout("block_causal", 17, 1, 1)
    q, k, v, *_ = _rand(17, d=16, seed=4)
    o, _, _ = attn_jvp_ref(q, k, v, *_rand(17, d=16, seed=5)[:3], m)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(a) for a in (q, k, v)), is_causal=True).numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("mask", LAYOUTS[1:4], ids=IDS[1:4])
def test_brute_force_elementwise(mask):
    """Per-element loops over the element predicate (not the key ranges)."""
    L = mask.seq_len
    q, k, v, tq, tk, tv = _rand(L, d=3, B=1, H=1, seed=6)
    c = 0.5
    o, to, lse = attn_jvp_ref(q, k, v, tq, tk, tv, mask, scale=c)
    q, k, v, tq, tk, tv = (a[0, 0] for a in (q, k, v, tq, tk, tv))
    for i in range(L):
        J = [j for j in range(L) if allowed(mask, i, j)]
        s = {j: c * sum(q[i, t] * k[j, t] for t in range(3)) for j in J}
        ts = {j: c * sum(tq[i, t] * k[j, t] + q[i, t] * tk[j, t] for t in range(3)) for j in J}
        mx = max(s.values())
        z = sum(math.exp(s[j] - mx) for j in J)
        p = {j: math.exp(s[j] - mx) / z for j in J}
        mu = sum(p[j] * ts[j] for j in J)
        for t in range(3):
            assert abs(o[0, 0, i, t] - sum(p[j] * v[j, t] for j in J)) < 1e-12
            ref = sum(p[j] * (ts[j] - mu) * v[j, t] + p[j] * tv[j, t] for j in J)
            assert abs(to[0, 0, i, t] - ref) < 1e-12
        assert abs(lse[0, 0, i] - (mx + math.log(z))) < 1e-12


@pytest.mark.parametrize("mask", LAYOUTS, ids=IDS)
def test_invariants(mask):
    L = mask.seq_len
    q, k, v, tq, tk, tv = _rand(L, seed=7)
    t2 = _rand(L, seed=8)[3:]
    c = 0.3
    _, to1, _ = attn_jvp_ref(q, k, v, tq, tk, tv, mask, scale=c)
    _, to2, _ = attn_jvp_ref(q, k, v, *t2, mask, scale=c)
    a, b = 0.7, -1.9
    # linearity in (tq, tk, tv)
    _, to_lin, _ = attn_jvp_ref(q, k, v, *(a * x + b * y for x, y in zip((tq, tk, tv), t2)), mask, scale=c)
    np.testing.assert_allclose(to_lin, a * to1 + b * to2, rtol=1e-11, atol=1e-11)
    # tangent scaling
    _, to_s, _ = attn_jvp_ref(q, k, v, 3.5 * tq, 3.5 * tk, 3.5 * tv, mask, scale=c)
    np.testing.assert_allclose(to_s, 3.5 * to1, rtol=1e-12, atol=1e-12)
    # zero tangents give exactly zero
    z = np.zeros_like(q)
    _, to0, _ = attn_jvp_ref(q, k, v, z, z, z, mask, scale=c)
    assert np.all(to0 == 0)
    # tq = tk = 0: tO = P tV, i.e. attention applied to tv (library routine)
    _, to_v, _ = attn_jvp_ref(q, k, v, z, z, tv, mask, scale=c)
    np.testing.assert_allclose(to_v, _sdpa(q, k, tv, mask, c), rtol=1e-12, atol=1e-12)
    # shifting every key by u keeps O and tO, moves lse by c <q_i, u>
    u = np.random.default_rng(9).standard_normal(q.shape[-1])
    o1, _, lse1 = attn_jvp_ref(q, k, v, tq, tk, tv, mask, scale=c)
    o3, to3, lse3 = attn_jvp_ref(q, k + u, v, tq, tk, tv, mask, scale=c)
    np.testing.assert_allclose(o3, o1, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(to3, to1, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(lse3 - lse1, c * q @ u, rtol=1e-10, atol=1e-10)
    # identical values and tv = 0: O = that value, tO = 0
    vc = np.broadcast_to(np.arange(q.shape[-1], dtype=float), q.shape).copy()
    o4, to4, _ = attn_jvp_ref(q, k, vc, tq, tk, z, mask, scale=c)
    np.testing.assert_allclose(o4, vc, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(to4, 0, atol=1e-11)


@pytest.mark.parametrize("mask", LAYOUTS[1:], ids=IDS[1:])
def test_masked_out_keys_change_nothing(mask):
    L = mask.seq_len
    q, k, v, tq, tk, tv = _rand(L, seed=10)
    rng = np.random.default_rng(11)
    for i in range(L):
        # evaluate the row alone on both sides so BLAS blocking is identical
        o, to, lse = attn_jvp_ref(q, k, v, tq, tk, tv, mask, rows=[i])
        blocked = [j for j in range(L) if not allowed(mask, i, j)]
        if not blocked:
            continue
        k2, v2, tk2, tv2 = (a.copy() for a in (k, v, tk, tv))
        for a in (k2, v2, tk2, tv2):
            a[:, :, blocked] += 5.0 * rng.standard_normal(a[:, :, blocked].shape)
        o2, to2, lse2 = attn_jvp_ref(q, k2, v2, tq, tk2, tv2, mask, rows=[i])
        np.testing.assert_array_equal(o2, o)
        np.testing.assert_array_equal(to2, to)
        np.testing.assert_array_equal(lse2, lse)


def test_teacher_forcing_clean_rows_have_zero_tangent():
    m = MaskLayout("tf_clean_noisy", 3, 4, 1)
    q, k, v, tq, tk, tv = _rand(m.seq_len, seed=12)
    n = m.half_len
    for t in (tq, tk, tv):
        t[:, :, :n] = 0
    _, to, _ = attn_jvp_ref(q, k, v, tq, tk, tv, m)
    assert np.all(to[:, :, :n] == 0)
    assert np.abs(to[:, :, n:]).max() > 0


def test_rows_without_allowed_keys():
    m = RectMask(6, ((0, 3, 0, 3), (4, 6, 0, 6)))   # row 3 has no allowed key
    q, k, v, tq, tk, tv = _rand(6, seed=13)
    o, to, lse = attn_jvp_ref(q, k, v, tq, tk, tv, m)
    assert np.all(o[:, :, 3] == 0) and np.all(to[:, :, 3] == 0) and np.all(np.isneginf(lse[:, :, 3]))
    assert np.all(np.isfinite(lse[:, :, [0, 1, 2, 4, 5]]))


def test_row_subset_matches_full_evaluation():
    m = MaskLayout("tf_clean_noisy", 3, 4, 1)
    x = _rand(m.seq_len, seed=14)
    o, to, lse = attn_jvp_ref(*x, m)
    rows = [23, 0, 5, 12, 13, 5]
    o2, to2, lse2 = attn_jvp_ref(*x, m, rows=rows)
    np.testing.assert_allclose(o2, o[:, :, rows], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(to2, to[:, :, rows], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse2, lse[:, :, rows], rtol=1e-13, atol=1e-13)
