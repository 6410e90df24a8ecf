"""Tangent-free token ranges in the mask descriptor (CPU only).

A descriptor derived with attn_jvp_mask_desc_tangent_free classifies every
visited (query tile, key tile) pair by which tangents it carries.  The
expected classes and per-class pair counts are computed here from the
oracle's element predicate and per-row key ranges, independently of the C++
builder.
"""
import numpy as np
import pytest

import attention_jvp_causal_amd as aj
from oracle.masks import MaskLayout, RectMask, dense_mask, key_ranges, unmasked_pairs

TM, TN = 128, 64


def _free_tokens(L, ranges):
    free = np.zeros(L, dtype=bool)
    for a, b in ranges:
        free[a:b] = True
    return free


def _expected(dm, free):
    """(variant per visited tile, pairs per class) from a dense mask.  A tile's
    variant is decided by the tokens that take part in it: the keys that some
    query of the tile may attend, and the queries that attend one of them
    (masked pairs contribute nothing, whatever their tangents)."""
    L = dm.shape[0]
    nq, nk = -(-L // TM), -(-L // TN)
    var = {}
    pairs = [0, 0, 0]
    for qt in range(nq):
        block = dm[qt * TM:(qt + 1) * TM]
        for kt in range(nk):
            sub = block[:, kt * TN:(kt + 1) * TN]
            cnt = int(sub.sum())
            if cnt == 0:
                continue
            keys = kt * TN + np.flatnonzero(sub.any(axis=0))
            rows = qt * TM + np.flatnonzero(sub.any(axis=1))
            kf, qf = bool(free[keys].all()), bool(free[rows].all())
            v = 3 if (qf and kf) else (1 if kf else 0)
            var[(qt, kt)] = v
            pairs[{0: 0, 1: 1, 3: 2}[v]] += cnt
    return var, pairs


CASES = [
    # mask, tangent-free ranges
    (MaskLayout("tf_clean_noisy", 4, 45, 1), [(0, 180)]),            # clean half, ragged boundary
    (MaskLayout("tf_clean_noisy", 3, 128, 1), [(0, 384)]),           # tile-aligned boundary
    (MaskLayout("block_causal", 7, 37, 3), [(0, 64), (100, 250)]),
    (MaskLayout("full", 3, 70, 1), [(0, 210)]),                      # everything tangent-free
    (MaskLayout("block_causal", 5, 61, 1), []),                      # nothing declared
    (RectMask(300, ((0, 300, 0, 100), (100, 300, 100, 300))), [(10, 20), (0, 15), (128, 300)]),
]


@pytest.mark.parametrize("mask,ranges", CASES)
@pytest.mark.parametrize("head_dim", [128, 64])
def test_variants_and_pair_counts_exhaustive(mask, ranges, head_dim):
    L = mask.seq_len
    if isinstance(mask, MaskLayout):
        base = aj.attn_jvp_mask_desc_build(mask.kind, mask.num_frames, mask.frame_tokens, mask.frames_per_chunk,
                                           head_dim=head_dim, dtype="bf16")
    else:
        base = aj.attn_jvp_mask_desc_from_rects(L, mask.rects, head_dim=head_dim, dtype="bf16")
    d = aj.attn_jvp_mask_desc_tangent_free(base, ranges)
    st, st0 = d.stats(), base.stats()
    # same mask: same pair count, tile kinds and bitmasks as the base
    for key in ("unmasked_pairs", "full_tiles", "partial_tiles", "num_q_tiles", "num_k_tiles"):
        assert st[key] == st0[key]
    dm = dense_mask(mask)
    var, pairs = _expected(dm, _free_tokens(L, ranges))
    for qt in range(st["num_q_tiles"]):
        for kt in range(st["num_k_tiles"]):
            assert d.tile_kind(qt, kt) == base.tile_kind(qt, kt)
            assert d.tile_variant(qt, kt) == var.get((qt, kt), -1), (qt, kt)
            if d.tile_kind(qt, kt) == 1:
                for r in (0, 1, 63, 127):
                    assert d.row_bits(qt, kt, r) == base.row_bits(qt, kt, r)
    assert list(d.work()) == pairs
    assert sum(pairs) == unmasked_pairs(mask)
    assert base.work() == (unmasked_pairs(mask), 0, 0)


def test_teacher_forcing_full_size_clean_context():
    # packed [clean | noisy] at the Wan2.1 shape, clean tokens declared
    # tangent-free: per-class pair counts from per-row key ranges, tile by
    # tile (the rows of a query tile fall into a few groups with the same key
    # ranges; per group and key tile, the allowed keys and how many of them
    # carry a tangent follow from prefix counts)
    T, F = 21, 1560
    m = MaskLayout("tf_clean_noisy", T, F, 1)
    L, half = m.seq_len, T * F
    base = aj.attn_jvp_mask_desc_build("tf_clean_noisy", T, F, 1, head_dim=128, dtype="bf16")
    d = aj.attn_jvp_mask_desc_tangent_free(base, [(0, half)])
    free = _free_tokens(L, [(0, half)])
    nk = -(-L // TN)
    k0s = np.arange(nk) * TN
    k1s = np.minimum(k0s + TN, L)
    NF = np.concatenate([[0], np.cumsum(~free)])  # keys carrying a tangent before index
    pairs = [0, 0, 0]
    for qt in range(-(-L // TM)):
        groups = {}
        for i in range(qt * TM, min(L, qt * TM + TM)):
            groups.setdefault(tuple(key_ranges(m, i)), []).append(i)
        allowed = np.zeros(nk, np.int64)        # allowed pairs per key tile
        tangent_keys = np.zeros(nk, np.int64)   # allowed keys carrying a tangent (summed over groups)
        tangent_rows = np.zeros(nk, bool)       # some attending row carries a tangent
        for rng, rows in groups.items():
            per_row = np.zeros(nk, np.int64)
            for a, b in rng:
                lo, hi = np.maximum(a, k0s), np.minimum(b, k1s)
                per_row += np.clip(hi - lo, 0, None)
                tangent_keys += np.where(hi > lo, NF[np.maximum(hi, lo)] - NF[lo], 0)
            allowed += per_row * len(rows)
            tangent_rows |= (per_row > 0) & (not free[rows].all())
        for kt in np.flatnonzero(allowed):
            kf, rf = tangent_keys[kt] == 0, not tangent_rows[kt]
            pairs[2 if (kf and rf) else 1 if kf else 0] += int(allowed[kt])
    assert list(d.work()) == pairs
    assert sum(pairs) == unmasked_pairs(m) == 1_124_323_200
    # the clean half is mostly primal-only work; noisy queries over clean keys
    # skip the key-tangent products
    assert pairs[2] > 0.45 * sum(pairs) and pairs[1] > 0.4 * sum(pairs)


def test_overlapping_ranges_merge():
    base = aj.attn_jvp_mask_desc_build("block_causal", 6, 50, 2, head_dim=128, dtype="bf16")
    a = aj.attn_jvp_mask_desc_tangent_free(base, [(0, 100), (50, 200), (199, 256)])
    b = aj.attn_jvp_mask_desc_tangent_free(base, [(0, 256)])
    st = a.stats()
    assert a.work() == b.work()
    for qt in range(st["num_q_tiles"]):
        for kt in range(st["num_k_tiles"]):
            assert a.tile_variant(qt, kt) == b.tile_variant(qt, kt)


@pytest.mark.parametrize("ranges", [[(5, 5)], [(10, 4)], [(-1, 3)], [(0, 301)]])
def test_invalid_ranges_rejected(ranges):
    base = aj.attn_jvp_mask_desc_build("full", 3, 100, 1, head_dim=128, dtype="bf16")
    with pytest.raises(aj.AttnJvpError) as e:
        aj.attn_jvp_mask_desc_tangent_free(base, ranges)
    assert e.value.status == aj.AJ_EINVAL
