"""Readers for the hand-written fixtures under tests/golden/."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_frame_grids():
    out = []
    cur = None
    with open(os.path.join(GOLDEN, "mask_frame_grids.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("layout"):
                _, kind, T, c = line.split()
                cur = [kind, int(T), int(c), []]
                out.append(cur)
            else:
                cur[3].append([int(ch) for ch in line])
    return [(k, T, c, np.array(rows, dtype=np.int64)) for k, T, c, rows in out]


def read_pair_counts():
    out = []
    with open(os.path.join(GOLDEN, "pair_counts.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            kind, T, F, c, n = line.split()
            out.append((kind, int(T), int(F), int(c), int(n)))
    return out
