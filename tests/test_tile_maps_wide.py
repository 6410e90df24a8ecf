"""The descriptor's 128-row and 256-row query-tile maps and its column map
against the oracle's element predicate (CPU only).

The 256-row map drives the primal forward at head_dim 128 and is not visible
through the C ABI, so a small test helper (tests/tile_map_dump.cpp) links the
library's own builder and prints its maps.  Every (query tile, key tile) is
checked: absent when no pair is allowed, full only when every in-range pair is
allowed, partial tiles with the exact per-row key bitmask, and every query tile
in the task order once ("Causal-rCM", App. B, sparse custom-mask
representation: tasks stream only the key ranges their rows may use).
"""
import shutil
import subprocess

import numpy as np
import pytest

from oracle.masks import MaskLayout, RectMask, dense_mask
from tilemap_util import build_dump_tool, check_all_maps, parse_maps, tile_input

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")


@pytest.fixture(scope="module")
def dump_tool(tmp_path_factory):
    return build_dump_tool(str(tmp_path_factory.mktemp("tilemap") / "tile_map_dump"))


def _maps(exe, inp):
    return parse_maps(subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout)


LAYOUTS = [("block_causal", 11, 61, 3), ("tf_clean_noisy", 5, 57, 1), ("block_causal", 9, 130, 1), ("full", 2, 300, 1)]


@pytest.mark.parametrize("kind,T,F,c", LAYOUTS)
def test_layouts_all_maps(dump_tool, kind, T, F, c):
    m = MaskLayout(kind, T, F, c)
    L = m.seq_len
    dm = dense_mask(m)
    code = {"full": 0, "block_causal": 1, "tf_clean_noisy": 2}[kind]
    maps = _maps(dump_tool, tile_input(("L", code, T, F, c)))
    check_all_maps(maps, dm, L, L)


def test_random_rectangles_all_maps(dump_tool):
    rng = np.random.default_rng(7)
    for trial in range(6):
        lq, lk = int(rng.integers(200, 900)), int(rng.integers(150, 700))
        rects, tries = [], 0
        occ = np.zeros((lq, lk), bool)
        while len(rects) < 6 and tries < 200:
            tries += 1
            q0, k0 = int(rng.integers(0, lq - 1)), int(rng.integers(0, lk - 1))
            q1, k1 = int(rng.integers(q0 + 1, lq + 1)), int(rng.integers(k0 + 1, lk + 1))
            if occ[q0:q1, k0:k1].any():
                continue
            occ[q0:q1, k0:k1] = True
            rects.append((q0, q1, k0, k1))
        dm = dense_mask(RectMask(lq, tuple(rects), kv_len=lk))
        maps = _maps(dump_tool, tile_input(("R", lq, lk, rects)))
        check_all_maps(maps, dm, lq, lk)
