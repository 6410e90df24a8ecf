"""Builds and runs tests/tile_map_dump.cpp (the library's own descriptor builder
behind a text interface) and checks the tile maps it prints against the
oracle's element predicate ("Causal-rCM", App. B, sparse custom-mask
representation: a query tile streams only the key tiles its rows may use, full
tiles without a mask, partial tiles with per-row key bitmasks)."""
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "attention_jvp_causal_amd", "csrc")

TILE_N = 64
# tile variants of the 128-row map (which tangents a tile carries)
TILE_JVP, TILE_KEYS_FREE, TILE_ALL_FREE = 0, 1, 3


def build_dump_tool(exe, extra_flags=()):
    """Compiles the helper and the library's builder with g++ into ``exe``."""
    subprocess.run(["g++", "-std=c++17", "-O1", *extra_flags, f"-I{CSRC}", f"-I{os.path.join(ROOT, 'include')}",
                    os.path.join(HERE, "tile_map_dump.cpp"), os.path.join(CSRC, "mask_desc.cpp"), "-o", exe],
                   check=True, capture_output=True)
    return exe


def parse_maps(text):
    """The maps printed by the helper: a list of dicts (rows, n_qt, n_kt, entries, tasks, split)."""
    out = text.split("\n")
    maps, i, cur = [], 0, None
    while i < len(out):
        t = out[i].split()
        i += 1
        if not t:
            continue
        if t[0] == "M":
            cur = {"rows": int(t[1]), "n_qt": int(t[2]), "n_kt": int(t[3]), "entries": [], "tasks": None, "split": None}
            maps.append(cur)
        elif t[0] == "E":
            qt, kt0, kt1, pidx, flags = map(int, t[1:6])
            bits = None
            if pidx >= 0:
                bits = [int(x, 16) for x in out[i:i + cur["rows"]]]
                i += cur["rows"]
            cur["entries"].append((qt, kt0, kt1, pidx, bits, flags))
        elif t[0] == "T":
            cur["tasks"] = [int(x) for x in t[1:]]
        elif t[0] == "S":
            cur["split"] = (int(t[1]), [int(x) for x in t[2:]])
    return maps


def tile_input(kind_or_rects, tf_ranges=()):
    """Helper stdin for a layout ("L", kind code, T, F, c) or rectangles ("R", lq, lk, rects)."""
    if kind_or_rects[0] == "L":
        s = "L " + " ".join(map(str, kind_or_rects[1:])) + "\n"
    else:
        _, lq, lk, rects = kind_or_rects
        s = f"R {lq} {lk} {len(rects)}\n" + "".join(" ".join(map(str, r)) + "\n" for r in rects)
    if tf_ranges:
        s += f"F {len(tf_ranges)}\n" + "".join(f"{a} {b}\n" for a, b in tf_ranges)
    return s


def check_map(m, dm, lo, lv, free=None):
    """Every (owner tile, visited tile) of map ``m`` against the dense predicate ``dm``
    ([lo, lv] booleans, owners on the first axis): absent when no pair is allowed, full
    only when every in-range pair is, partial tiles with the exact per-row bitmask,
    every owner tile once in the task order.  ``free``: per-token booleans of the
    declared tangent-free tokens (checks the tile variants: keys free when every
    key that some row of the tile may attend is free, rows free when every row
    attending one of them is), or None (no variants)."""
    tm, tn = m["rows"], TILE_N
    assert m["n_qt"] == -(-lo // tm) and m["n_kt"] == -(-lv // tn)
    assert sorted(m["tasks"]) == list(range(m["n_qt"]))
    seen = {}
    for qt, kt0, kt1, pidx, bits, flags in m["entries"]:
        assert kt0 < kt1
        if pidx >= 0:
            assert kt1 == kt0 + 1
        for kt in range(kt0, kt1):
            assert (qt, kt) not in seen
            seen[(qt, kt)] = (bits, flags)
    for qt in range(m["n_qt"]):
        r0, r1 = qt * tm, min(lo, qt * tm + tm)
        for kt in range(m["n_kt"]):
            k0, k1 = kt * tn, min(lv, kt * tn + tn)
            block = dm[r0:r1, k0:k1]
            if (qt, kt) not in seen:
                assert not block.any(), (tm, qt, kt)
                continue
            bits, flags = seen[(qt, kt)]
            if free is None:
                assert flags == TILE_JVP, (tm, qt, kt, flags)
            else:  # decided by the keys some row may attend and the rows attending one of them
                kf = bool(free[k0 + np.flatnonzero(block.any(axis=0))].all())
                qf = bool(free[r0 + np.flatnonzero(block.any(axis=1))].all())
                want = (TILE_ALL_FREE if qf else TILE_KEYS_FREE) if kf else TILE_JVP
                assert flags == want, (tm, qt, kt, flags, want)
            if bits is None:  # full: every in-range pair allowed, tile inside the key range
                assert block.all() and kt * tn + tn <= lv, (tm, qt, kt)
            else:
                for row in range(tm):
                    i = r0 + row
                    want = 0
                    if i < lo:
                        for j in range(k0, k1):
                            if dm[i, j]:
                                want |= 1 << (j - k0)
                    assert bits[row] == want, (tm, qt, kt, row)
    if m["split"] is not None:
        n_primal, order = m["split"]
        assert sorted(order) == list(range(m["n_qt"]))
        primal_only = [all(f == TILE_ALL_FREE for q, _, _, _, _, f in m["entries"] if q == qt) for qt in range(m["n_qt"])]
        assert [primal_only[qt] for qt in order] == [True] * n_primal + [False] * (m["n_qt"] - n_primal)


def check_all_maps(maps, dm, lq, lk, free=None):
    """The three maps of a descriptor: 128-row query tiles (with variants), 256-row
    query tiles and 128-key column tiles of the transposed mask (no variants)."""
    assert [x["rows"] for x in maps] == [128, 256, 128]
    check_map(maps[0], dm, lq, lk, free)
    check_map(maps[1], dm, lq, lk)
    check_map(maps[2], dm.T, lk, lq)
