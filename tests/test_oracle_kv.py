"""Pins for the oracle's query-chunk-over-KV-cache masks (CPU only).

A rectangular mask (queries and keys of different lengths) is pinned against
PyTorch's scaled_dot_product_attention with the same boolean mask, and a
chunk attending a cache prefix (Sec. 3.2.1 "KV Cache", readonly mode) against
the rows of that chunk in the block-causal layout of the whole sequence
(Sec. 2.3: a chunk sees every earlier chunk and itself).
"""
import numpy as np
import pytest
import torch

from oracle import MaskLayout, RectMask, attn_jvp_ref, chunk_over_cache, dense_mask, unmasked_pairs


def _rand(shape, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal(shape) for _ in range(3)]


@pytest.mark.parametrize("Lq,Lk,rects", [
    (5, 12, ((0, 5, 0, 12),)),
    (7, 19, ((0, 3, 0, 10), (3, 7, 2, 19))),
    (6, 4, ((0, 6, 0, 4),)),
])
def test_rectangular_mask_matches_sdpa(Lq, Lk, rects):
    m = RectMask(Lq, rects, kv_len=Lk)
    d = 8
    q, = _rand((1, 2, Lq, d), 1)[:1]
    k, v = _rand((1, 2, Lk, d), 2)[:2]
    z = np.zeros_like(q)
    zk = np.zeros_like(k)
    o, to, lse = attn_jvp_ref(q, k, v, z, zk, zk, m, scale=0.3)
    dm = torch.from_numpy(dense_mask(m))
    assert dm.shape == (Lq, Lk)
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=dm, scale=0.3).numpy()
    np.testing.assert_allclose(o, want, rtol=1e-12, atol=1e-13)
    assert not to.any()
    s = 0.3 * np.einsum("bhid,bhjd->bhij", q, k)
    s[..., ~dense_mask(m)] = -np.inf
    np.testing.assert_allclose(lse, np.log(np.exp(s).sum(-1)), rtol=1e-12)
    assert unmasked_pairs(m) == int(dense_mask(m).sum())


@pytest.mark.parametrize("T,F,c", [(6, 5, 2), (7, 4, 3), (4, 9, 1)])
def test_chunk_over_cache_equals_block_causal_rows(T, F, c):
    lay = MaskLayout("block_causal", T, F, c)
    L = lay.seq_len
    d = 8
    q, k, v = _rand((2, 2, L, d), 3)
    z = np.zeros_like(q)
    C = c * F
    for n in range(-(-T // c)):
        r0, r1 = n * C, min(L, (n + 1) * C)
        m = chunk_over_cache(r1 - r0, r0)
        o, _, lse = attn_jvp_ref(q[:, :, r0:r1], k[:, :, :r1], v[:, :, :r1], z[:, :, r0:r1], z[:, :, :r1],
                                 z[:, :, :r1], m)
        ow, _, lsew = attn_jvp_ref(q, k, v, z, z, z, lay, rows=range(r0, r1))
        np.testing.assert_allclose(o, ow, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse, lsew, rtol=1e-12, atol=1e-13)
