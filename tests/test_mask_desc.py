"""The C++ mask descriptor against the oracle's element predicate (CPU only).

The descriptor is built by the product library; the predicate and the key
ranges come from oracle/masks.py, written independently from the pages.
"""
import numpy as np
import pytest

import attention_jvp_causal_amd as aj
from oracle.masks import MaskLayout, RectMask, dense_mask, key_ranges, unmasked_pairs
from golden_io import read_pair_counts

SMALL = [
    ("full", 3, 70, 1),
    ("block_causal", 5, 61, 1),      # frames not tile aligned, ragged L
    ("block_causal", 7, 37, 3),      # ragged last chunk
    ("block_causal", 2, 64, 1),      # tile-aligned frames
    ("tf_clean_noisy", 4, 45, 1),
    ("tf_clean_noisy", 5, 33, 2),
]


def _bits_from_dense(dm, qt, kt, row, tm=128, tn=64):
    i = qt * tm + row
    L = dm.shape[0]
    if i >= L:
        return 0
    b = 0
    for j in range(tn):
        key = kt * tn + j
        if key < L and dm[i, key]:
            b |= 1 << j
    return b


@pytest.mark.parametrize("kind,T,F,c", SMALL)
@pytest.mark.parametrize("head_dim,dtype", [(128, "bf16"), (64, "bf16"), (64, "f32")])
def test_small_layouts_exhaustive(kind, T, F, c, head_dim, dtype):
    m = MaskLayout(kind, T, F, c)
    d = aj.attn_jvp_mask_desc_build(kind, T, F, c, head_dim=head_dim, dtype=dtype)
    st = d.stats()
    L = m.seq_len
    assert st["seq_len"] == L and st["unmasked_pairs"] == unmasked_pairs(m)
    dm = dense_mask(m)
    tm, tn = st["tile_m"], st["tile_n"]
    full = partial = 0
    for qt in range(st["num_q_tiles"]):
        for kt in range(st["num_k_tiles"]):
            kind_ = d.tile_kind(qt, kt)
            bits = [_bits_from_dense(dm, qt, kt, r, tm, tn) for r in range(tm)]
            got = [d.row_bits(qt, kt, r) for r in range(tm)]
            valid_rows = min(tm, L - qt * tm)
            if kind_ == 2:
                full += 1
                # full: every valid row sees all 64 keys, all keys in range
                assert all(b == (1 << tn) - 1 for b in bits[:valid_rows])
                assert all(g == (1 << 64) - 1 for g in got[:valid_rows])
            elif kind_ == 1:
                partial += 1
                assert got == bits
                assert any(bits) and not all(b == (1 << tn) - 1 for b in bits[:valid_rows])
            else:
                assert not any(bits)
    assert full == st["full_tiles"] and partial == st["partial_tiles"]


@pytest.mark.parametrize("kind,T,F,c,n", read_pair_counts())
def test_full_size_pair_counts_and_sampled_tiles(kind, T, F, c, n):
    m = MaskLayout(kind, T, F, c)
    d = aj.attn_jvp_mask_desc_build(kind, T, F, c, head_dim=128, dtype="bf16")
    st = d.stats()
    assert st["unmasked_pairs"] == n
    # full tiles hold exactly 128 x 64 allowed pairs unless the last query tile
    # is ragged; partial tiles the rest
    rng = np.random.default_rng(0)
    tm, tn, L = st["tile_m"], st["tile_n"], st["seq_len"]
    for _ in range(60):
        qt = int(rng.integers(st["num_q_tiles"]))
        kt = int(rng.integers(st["num_k_tiles"]))
        kind_ = d.tile_kind(qt, kt)
        for r in list(rng.integers(0, tm, size=6)) + [0, tm - 1]:
            i = qt * tm + int(r)
            want = 0
            if i < L:
                for a, b in key_ranges(m, i):
                    lo, hi = max(a, kt * tn), min(b, kt * tn + tn)
                    if lo < hi:
                        want |= ((1 << (hi - lo)) - 1) << (lo - kt * tn)
            got = d.row_bits(qt, kt, int(r))
            if kind_ == 2 and i < L:
                assert want == (1 << tn) - 1
            assert got == want or (kind_ == 2 and i < L and got == (1 << 64) - 1)


def test_tasks_cover_every_query_tile_longest_first():
    # visited-tile counts per query tile via the public tile map
    d = aj.attn_jvp_mask_desc_build("tf_clean_noisy", 3, 100, 1, head_dim=64, dtype="bf16")
    st = d.stats()
    work = [sum(d.tile_kind(qt, kt) > 0 for kt in range(st["num_k_tiles"])) for qt in range(st["num_q_tiles"])]
    assert sum(work) == st["full_tiles"] + st["partial_tiles"]


@pytest.mark.parametrize("rects,L", [
    ([(0, 5, 0, 5), (5, 200, 0, 3), (5, 200, 70, 200), (90, 140, 4, 69)], 200),
    ([(0, 300, 0, 300)], 300),
    ([], 50),
    ([(10, 11, 64, 128)], 130),
])
def test_from_rects_matches_rect_predicate(rects, L):
    m = RectMask(L, tuple(rects))
    d = aj.attn_jvp_mask_desc_from_rects(L, rects, head_dim=128, dtype="bf16")
    st = d.stats()
    assert st["unmasked_pairs"] == unmasked_pairs(m)
    dm = dense_mask(m)
    for qt in range(st["num_q_tiles"]):
        for kt in range(st["num_k_tiles"]):
            kind_ = d.tile_kind(qt, kt)
            for r in range(128):
                want = _bits_from_dense(dm, qt, kt, r)
                got = d.row_bits(qt, kt, r)
                if kind_ == 2 and qt * 128 + r < L:
                    assert want == (1 << 64) - 1
                else:
                    assert got == want


def test_equivalent_rects_give_same_tile_map():
    a = aj.attn_jvp_mask_desc_build("block_causal", 6, 50, 2, head_dim=128, dtype="bf16")
    rects = [(0, 100, 0, 100), (100, 200, 0, 200), (200, 300, 0, 300)]
    b = aj.attn_jvp_mask_desc_from_rects(300, rects, head_dim=128, dtype="bf16")
    assert a.stats() == b.stats()


@pytest.mark.parametrize("mask", [
    MaskLayout("block_causal", 7, 37, 3), MaskLayout("tf_clean_noisy", 4, 45, 1), MaskLayout("full", 3, 70, 1),
    RectMask(300, ((0, 100, 0, 100), (130, 300, 0, 40), (130, 300, 150, 300))),
], ids=["c3_ragged", "tf", "full", "rects"])
def test_column_map_is_the_transposed_mask(mask):
    # the key-tile map (128 keys x 64 queries) against the element predicate
    L = mask.seq_len
    if isinstance(mask, MaskLayout):
        d = aj.attn_jvp_mask_desc_build(mask.kind, mask.num_frames, mask.frame_tokens, mask.frames_per_chunk,
                                        head_dim=128, dtype="bf16")
    else:
        d = aj.attn_jvp_mask_desc_from_rects(L, mask.rects, head_dim=128, dtype="bf16")
    dm = dense_mask(mask)
    nk, nq = -(-L // 128), -(-L // 64)
    pairs = 0
    for kt in range(nk):
        for qt in range(nq):
            for r in range(128):
                key = kt * 128 + r
                want = 0
                if key < L:
                    for j in range(64):
                        q = qt * 64 + j
                        if q < L and dm[q, key]:
                            want |= 1 << j
                got = d.col_bits(kt, qt, r)
                assert got == want, (kt, qt, r)
                pairs += bin(got).count("1")
    assert pairs == unmasked_pairs(mask)


@pytest.mark.parametrize("Lq,Lk,rects", [
    (300, 1000, ((0, 300, 0, 1000),)),
    (130, 70, ((0, 60, 0, 70), (60, 130, 5, 66))),
    (200, 4680, ((0, 100, 0, 4000), (100, 200, 0, 4680))),
])
def test_kv_descriptor_maps(Lq, Lk, rects):
    m = RectMask(Lq, rects, kv_len=Lk)
    d = aj.attn_jvp_mask_desc_from_rects_kv(Lq, Lk, rects, head_dim=128, dtype="bf16")
    st = d.stats()
    assert st["seq_len"] == Lq and st["kv_len"] == Lk and st["unmasked_pairs"] == unmasked_pairs(m)
    assert st["num_q_tiles"] == -(-Lq // 128) and st["num_k_tiles"] == -(-Lk // 64)
    dm = dense_mask(m)
    rng = np.random.default_rng(1)
    for _ in range(40):
        qt, kt = int(rng.integers(st["num_q_tiles"])), int(rng.integers(st["num_k_tiles"]))
        for r in (0, 5, 127, int(rng.integers(128))):
            i = qt * 128 + r
            want = 0
            if i < Lq:
                for j in range(64):
                    if kt * 64 + j < Lk and dm[i, kt * 64 + j]:
                        want |= 1 << j
            got = d.row_bits(qt, kt, r)
            if d.tile_kind(qt, kt) == 2 and i < Lq:
                assert want == (1 << 64) - 1
            else:
                assert got == want
        kk, qq = int(rng.integers(-(-Lk // 128))), int(rng.integers(-(-Lq // 64)))
        for r in (0, 77, 127):
            key = kk * 128 + r
            want = 0
            if key < Lk:
                for j in range(64):
                    if qq * 64 + j < Lq and dm[qq * 64 + j, key]:
                        want |= 1 << j
            assert d.col_bits(kk, qq, r) == want


def test_kv_descriptor_errors():
    with pytest.raises(aj.AttnJvpError) as e:
        aj.attn_jvp_mask_desc_from_rects_kv(10, 20, [(0, 10, 0, 21)], head_dim=128, dtype="bf16")
    assert e.value.status == aj.AJ_EMASK
    d = aj.attn_jvp_mask_desc_from_rects_kv(10, 20, [(0, 10, 0, 20)], head_dim=128, dtype="bf16")
    with pytest.raises(aj.AttnJvpError) as e:
        aj.attn_jvp_mask_desc_tangent_free(d, [(0, 5)])
    assert e.value.status == aj.AJ_EINVAL
