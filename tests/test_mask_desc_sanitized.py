"""The host-side descriptor builder under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

tests/tile_map_dump.cpp links the library's own builder (mask_desc.cpp); here
both are compiled with g++ ``-fsanitize=address,undefined`` and driven over
frame layouts, rectangles with query and key lengths apart (the KV-cache form),
tangent-free token ranges (overlapping, touching the ends, covering
everything), the full-size workload layouts, and inputs the builder must
reject.  Every run must end without a sanitizer report; valid inputs must give
tile maps that agree with the oracle's element predicate and variants that
agree with the declared tangent-free tokens ("Causal-rCM", App. B, sparse
custom-mask representation; Sec. 3.1.2, the clean context carries no tangent).
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle.masks import MaskLayout, RectMask, dense_mask
from tilemap_util import build_dump_tool, check_all_maps, parse_maps, tile_input

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")

KIND = {"full": 0, "block_causal": 1, "tf_clean_noisy": 2}
AJ_EINVAL, AJ_EMASK = 1, 5
SAN_FLAGS = ("-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g")


_ASAN = {"options": "detect_leaks=1:abort_on_error=0"}


@pytest.fixture(scope="module")
def san_tool(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("tilemap_san") / "tile_map_dump_san")
    try:
        build_dump_tool(exe, SAN_FLAGS)
    except subprocess.CalledProcessError as e:  # no sanitizer runtime in this toolchain
        pytest.skip("g++ cannot build with -fsanitize=address,undefined: " + e.stderr.decode()[-300:])
    # LeakSanitizer needs ptrace; where the sandbox denies it, keep the other checks
    r = subprocess.run([exe], input="L 0 1 1 1\n", capture_output=True, text=True,
                       env=dict(os.environ, ASAN_OPTIONS=_ASAN["options"]), timeout=120)
    if "LeakSanitizer has encountered a fatal error" in r.stderr:
        _ASAN["options"] = "detect_leaks=0:abort_on_error=0"
    return exe


def _run(exe, inp):
    env = dict(os.environ, ASAN_OPTIONS=_ASAN["options"], UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], input=inp, capture_output=True, text=True, env=env, timeout=600)
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-3000:]
    return r


def _ok(exe, inp):
    r = _run(exe, inp)
    assert r.returncode == 0, (r.returncode, r.stdout[-300:], r.stderr[-300:])
    return parse_maps(r.stdout)


def _free_mask(L, ranges):
    f = np.zeros(L, bool)
    for a, b in ranges:
        f[a:b] = True
    return f


@pytest.mark.parametrize("kind,T,F,c,tf", [
    ("tf_clean_noisy", 5, 57, 1, "clean"),
    ("tf_clean_noisy", 4, 100, 2, "clean"),
    ("block_causal", 7, 45, 3, "random"),
    ("block_causal", 3, 130, 1, "none"),
    ("full", 2, 200, 1, "all"),
    ("full", 1, 1, 1, "none"),
])
def test_layouts_with_tangent_free_ranges(san_tool, kind, T, F, c, tf):
    m = MaskLayout(kind, T, F, c)
    L = m.seq_len
    rng = np.random.default_rng(L)
    if tf == "clean":
        ranges = [(0, L // 2)]
    elif tf == "all":
        ranges = [(0, L)]
    elif tf == "random":  # overlapping, one touching each end
        ranges = [(0, int(rng.integers(1, L // 3)))]
        for _ in range(3):
            a = int(rng.integers(0, L - 1))
            ranges.append((a, int(rng.integers(a + 1, L + 1))))
        ranges.append((int(rng.integers(L // 2, L - 1)), L))
    else:
        ranges = []
    maps = _ok(san_tool, tile_input(("L", KIND[kind], T, F, c), ranges))
    check_all_maps(maps, dense_mask(m), L, L, _free_mask(L, ranges) if ranges else None)


def test_kv_and_square_rectangles(san_tool):
    rng = np.random.default_rng(11)
    for trial in range(8):
        square = trial % 2 == 0
        lq = int(rng.integers(1, 700))
        lk = lq if square else int(rng.integers(1, 900))
        rects, occ = [], np.zeros((lq, lk), bool)
        for _ in range(60):
            if len(rects) == 7:
                break
            q0, k0 = int(rng.integers(0, lq)), int(rng.integers(0, lk))
            q1, k1 = int(rng.integers(q0 + 1, lq + 1)), int(rng.integers(k0 + 1, lk + 1))
            if not occ[q0:q1, k0:k1].any():
                occ[q0:q1, k0:k1] = True
                rects.append((q0, q1, k0, k1))
        ranges = []
        if square and lq > 2:
            for _ in range(2):
                a = int(rng.integers(0, lq - 1))
                ranges.append((a, int(rng.integers(a + 1, lq + 1))))
        maps = _ok(san_tool, tile_input(("R", lq, lk, rects), ranges))
        dm = dense_mask(RectMask(lq, tuple(rects), kv_len=lk))
        check_all_maps(maps, dm, lq, lk, _free_mask(lq, ranges) if ranges else None)


@pytest.mark.parametrize("kind,T,F,c,clean_free", [
    ("block_causal", 21, 1560, 3, False),
    ("block_causal", 21, 1560, 1, False),
    ("tf_clean_noisy", 21, 1560, 1, True),
    ("block_causal", 21, 880, 3, False),
])
def test_full_size_layouts_run_clean(san_tool, kind, T, F, c, clean_free):
    L = T * F * (2 if kind == "tf_clean_noisy" else 1)
    maps = _ok(san_tool, tile_input(("L", KIND[kind], T, F, c), [(0, L // 2)] if clean_free else []))
    assert [x["rows"] for x in maps] == [128, 256, 128]
    for x in maps:
        assert sorted(x["tasks"]) == list(range(x["n_qt"]))
        for qt, kt0, kt1, pidx, bits, flags in x["entries"]:
            assert 0 <= qt < x["n_qt"] and 0 <= kt0 < kt1 <= x["n_kt"]
    if clean_free:  # every query tile inside the clean half attends only clean keys: primal-only
        n_primal, order = maps[0]["split"]
        assert n_primal == (L // 2) // 128


@pytest.mark.parametrize("inp,status", [
    (tile_input(("R", 100, 100, [(0, 50, 0, 60), (40, 100, 50, 100)])), AJ_EMASK),   # overlapping rectangles
    (tile_input(("R", 100, 80, [(0, 50, 0, 81)])), AJ_EMASK),                        # key range past kv_len
    (tile_input(("R", 100, 100, [(10, 10, 0, 5)])), AJ_EMASK),                       # empty rectangle
    (tile_input(("R", 100, 100, [(-1, 5, 0, 5)])), AJ_EMASK),                        # negative start
    (tile_input(("R", 100, 100, [(0, 100, 0, 100)]), [(0, 101)]), AJ_EINVAL),       # tangent-free range past L
    (tile_input(("R", 100, 100, [(0, 100, 0, 100)]), [(5, 5)]), AJ_EINVAL),         # empty tangent-free range
    (tile_input(("R", 100, 90, [(0, 100, 0, 90)]), [(0, 10)]), AJ_EINVAL),          # tangent-free ranges on a KV shape
    (tile_input(("R", 0, 10, [])), AJ_EINVAL),                                        # empty sequence
])
def test_rejected_inputs(san_tool, inp, status):
    r = _run(san_tool, inp)
    assert r.returncode == 1 and r.stdout.split() == ["ERR", str(status)], (r.returncode, r.stdout[-200:])


def test_rejected_layouts(san_tool):
    # no frames; no tokens; no frames per chunk; unknown layout kind
    for inp in ["L 1 0 10 1\n", "L 1 6 0 1\n", "L 1 3 10 0\n", "L 7 3 10 1\n"]:
        r = _run(san_tool, inp)
        assert r.returncode == 1 and not r.stdout.strip(), (inp, r.returncode, r.stdout[-200:])
