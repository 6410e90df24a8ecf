"""Pins for the oracle's mask layouts (oracle/masks.py)."""
import numpy as np
import pytest

from oracle.masks import MaskLayout, RectMask, allowed, dense_mask, frame_grid, key_ranges, unmasked_pairs
from golden_io import read_frame_grids, read_pair_counts


@pytest.mark.parametrize("kind,T,c,grid", read_frame_grids(),
                         ids=lambda x: str(x) if not isinstance(x, np.ndarray) else "grid")
def test_frame_grids_match_golden(kind, T, c, grid):
    # 3 tokens per frame so that "full inside a frame" is exercised too
    m = MaskLayout(kind, T, 3, c)
    assert np.array_equal(frame_grid(m), grid)
    # every token pair inherits its frames' entry
    dm = dense_mask(m)
    L = m.seq_len
    fr = np.arange(L) // 3
    assert np.array_equal(dm, grid[fr][:, fr].astype(bool))


@pytest.mark.parametrize("kind,T,F,c,n", read_pair_counts())
def test_pair_counts_closed_form(kind, T, F, c, n):
    m = MaskLayout(kind, T, F, c)
    assert unmasked_pairs(m) == n


@pytest.mark.parametrize("layout", [
    MaskLayout("full", 3, 5), MaskLayout("block_causal", 5, 3, 1), MaskLayout("block_causal", 5, 3, 2),
    MaskLayout("tf_clean_noisy", 4, 3, 1), MaskLayout("tf_clean_noisy", 5, 2, 2),
    RectMask(11, ((0, 4, 0, 4), (4, 11, 0, 2), (4, 11, 6, 11), (7, 9, 3, 5))),
])
def test_key_ranges_agree_with_predicate(layout):
    L = layout.seq_len
    for i in range(L):
        row = np.zeros(L, dtype=bool)
        for a, b in key_ranges(layout, i):
            assert 0 <= a < b <= L
            row[a:b] = True
        assert np.array_equal(row, [allowed(layout, i, j) for j in range(L)])


def test_frame_causal_is_token_causal_when_frames_are_single_tokens():
    m = MaskLayout("block_causal", 9, 1, 1)
    assert np.array_equal(dense_mask(m), np.tril(np.ones((9, 9), dtype=bool)))
