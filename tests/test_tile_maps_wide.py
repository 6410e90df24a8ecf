"""The descriptor's 128-row and 256-row query-tile maps against the oracle's
element predicate (CPU only).

The 256-row map drives the primal forward at head_dim 128 and is not visible
through the C ABI, so a small test helper (tests/tile_map_dump.cpp) links the
library's own builder and prints both maps.  Every (query tile, key tile) is
checked: absent when no pair is allowed, full only when every in-range pair is
allowed, partial tiles with the exact per-row key bitmask, and every query tile
in the task order once ("Causal-rCM", App. B, sparse custom-mask
representation: tasks stream only the key ranges their rows may use).
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle.masks import MaskLayout, RectMask, dense_mask

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "attention_jvp_causal_amd", "csrc")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")


@pytest.fixture(scope="module")
def dump_tool(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("tilemap") / "tile_map_dump")
    subprocess.run(["g++", "-std=c++17", "-O1", f"-I{CSRC}", f"-I{os.path.join(ROOT, 'include')}",
                    os.path.join(HERE, "tile_map_dump.cpp"), os.path.join(CSRC, "mask_desc.cpp"), "-o", exe],
                   check=True, capture_output=True)
    return exe


def _maps(exe, inp):
    out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout.split("\n")
    maps, i = [], 0
    while i < len(out):
        t = out[i].split()
        i += 1
        if not t:
            continue
        if t[0] == "M":
            cur = {"rows": int(t[1]), "n_qt": int(t[2]), "n_kt": int(t[3]), "entries": [], "tasks": None}
            maps.append(cur)
        elif t[0] == "E":
            qt, kt0, kt1, pidx = map(int, t[1:])
            bits = None
            if pidx >= 0:
                bits = [int(x, 16) for x in out[i:i + cur["rows"]]]
                i += cur["rows"]
            cur["entries"].append((qt, kt0, kt1, pidx, bits))
        elif t[0] == "T":
            cur["tasks"] = [int(x) for x in t[1:]]
    return maps


def _check(m, dm, lq, lk):
    tm, tn = m["rows"], 64
    assert m["n_qt"] == -(-lq // tm) and m["n_kt"] == -(-lk // tn)
    assert sorted(m["tasks"]) == list(range(m["n_qt"]))
    seen = {}
    for qt, kt0, kt1, pidx, bits in m["entries"]:
        assert kt0 < kt1
        if pidx >= 0:
            assert kt1 == kt0 + 1
        for kt in range(kt0, kt1):
            assert (qt, kt) not in seen
            seen[(qt, kt)] = bits
    for qt in range(m["n_qt"]):
        r0, r1 = qt * tm, min(lq, qt * tm + tm)
        for kt in range(m["n_kt"]):
            k0, k1 = kt * tn, min(lk, kt * tn + tn)
            block = dm[r0:r1, k0:k1]
            if (qt, kt) not in seen:
                assert not block.any(), (tm, qt, kt)
                continue
            bits = seen[(qt, kt)]
            if bits is None:  # full: every in-range pair allowed, tile inside the key range
                assert block.all() and kt * tn + tn <= lk, (tm, qt, kt)
            else:
                for row in range(tm):
                    i = r0 + row
                    want = 0
                    if i < lq:
                        for j in range(k0, k1):
                            if dm[i, j]:
                                want |= 1 << (j - k0)
                    assert bits[row] == want, (tm, qt, kt, row)


LAYOUTS = [("block_causal", 11, 61, 3), ("tf_clean_noisy", 5, 57, 1), ("block_causal", 9, 130, 1), ("full", 2, 300, 1)]


@pytest.mark.parametrize("kind,T,F,c", LAYOUTS)
def test_layouts_both_maps(dump_tool, kind, T, F, c):
    m = MaskLayout(kind, T, F, c)
    L = m.seq_len
    dm = dense_mask(m)
    code = {"full": 0, "block_causal": 1, "tf_clean_noisy": 2}[kind]
    maps = _maps(dump_tool, f"L {code} {T} {F} {c}\n")
    assert [x["rows"] for x in maps] == [128, 256]
    for x in maps:
        _check(x, dm, L, L)


def test_random_rectangles_both_maps(dump_tool):
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
        inp = f"R {lq} {lk} {len(rects)}\n" + "\n".join(" ".join(map(str, r)) for r in rects) + "\n"
        maps = _maps(dump_tool, inp)
        for x in maps:
            _check(x, dm, lq, lk)
