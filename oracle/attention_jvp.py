"""fp64 oracle: masked softmax attention and its forward-mode JVP.

Test infrastructure (see the package docstring).

Plain definition, per (batch, head), with c the softmax scale and A(i) the set
of keys query i may attend to ("Causal-rCM", App. B):

* scores        s_ij  = c * <q_i, k_j>                          (Eq. 42)
* score tangent ts_ij = c * (<tq_i, k_j> + <q_i, tk_j>)          (Eq. 43)
  The mask is a fixed routing object with no tangent; keys outside A(i) take
  no part in either the primal or the tangent.
* P_ij = exp(s_ij - m_i) / l_i over j in A(i), with m_i = max s_ij and
  l_i = sum exp(s_ij - m_i);  O_i = sum_j P_ij v_j;  lse_i = m_i + ln l_i
* mu_i  = sum_j P_ij ts_ij
  tO_i  = sum_j P_ij (ts_ij - mu_i) v_j + sum_j P_ij tv_j        (Eq. 44)

It is evaluated densely over each query group's allowed key ranges as an
ordinary two-pass softmax with numpy fp64 matrix products: no online softmax,
no tiles.  Rows with no allowed key give O = tO = 0 and lse = -inf (a reading:
the pages never meet such rows).  lse is not defined on the pages; the
FlashAttention convention (natural log, scale included) is used.
"""
from __future__ import annotations

from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

from .masks import key_ranges

_ROW_BLOCK = 256  # rows per dense block, bounds memory at ~L * 256 * 8 bytes per matrix


def _row_groups(mask, rows: Sequence[int]):
    """Group the requested rows by their allowed-key set (order of first use)."""
    groups = {}
    for i in rows:
        kr = tuple(key_ranges(mask, int(i)))
        groups.setdefault(kr, []).append(int(i))
    return [(g, list(kr)) for kr, g in groups.items()]


def _gather_keys(x: np.ndarray, ranges: List[Tuple[int, int]]) -> np.ndarray:
    if len(ranges) == 1:
        a, b = ranges[0]
        return x[a:b]
    return np.concatenate([x[a:b] for a, b in ranges], axis=0)


def attn_jvp_ref(q, k, v, tq, tk, tv, mask, scale: Optional[float] = None,
                 rows: Optional[Iterable[int]] = None):
    """Primal O, tangent tO and lse of masked attention, in float64.

    q, k, v, tq, tk, tv: arrays of shape [B, H, L, d] (upcast to float64).
    mask: a ``MaskLayout`` or ``RectMask`` (oracle.masks).
    rows: optional subset of query rows; outputs then have that many rows,
    in the given order.
    Returns (o [B,H,R,d], to [B,H,R,d], lse [B,H,R]).
    """
    q, k, v, tq, tk, tv = (np.asarray(a, dtype=np.float64) for a in (q, k, v, tq, tk, tv))
    B, H, L, d = q.shape
    c = 1.0 / np.sqrt(d) if scale is None else float(scale)
    rows = list(range(L)) if rows is None else [int(r) for r in rows]
    R = len(rows)
    pos = {}
    for n, r in enumerate(rows):
        pos.setdefault(r, []).append(n)

    o = np.zeros((B, H, R, d))
    to = np.zeros((B, H, R, d))
    lse = np.full((B, H, R), -np.inf)

    for grp, ranges in _row_groups(mask, rows):
        nk = sum(b - a for a, b in ranges)
        if nk == 0:
            continue  # no allowed key: O = tO = 0, lse = -inf
        for b_ in range(B):
            for h in range(H):
                K, TK = _gather_keys(k[b_, h], ranges), _gather_keys(tk[b_, h], ranges)
                V, TV = _gather_keys(v[b_, h], ranges), _gather_keys(tv[b_, h], ranges)
                for r0 in range(0, len(grp), _ROW_BLOCK):
                    blk = grp[r0:r0 + _ROW_BLOCK]
                    out_idx = [pos[r][0] for r in blk]
                    Q, TQ = q[b_, h, blk], tq[b_, h, blk]
                    s = c * (Q @ K.T)
                    ts = c * (TQ @ K.T + Q @ TK.T)
                    m = s.max(axis=1, keepdims=True)
                    e = np.exp(s - m)
                    l = e.sum(axis=1, keepdims=True)
                    P = e / l
                    mu = (P * ts).sum(axis=1, keepdims=True)
                    o[b_, h, out_idx] = P @ V
                    to[b_, h, out_idx] = (P * (ts - mu)) @ V + P @ TV
                    lse[b_, h, out_idx] = m[:, 0] + np.log(l[:, 0])
    # duplicated requested rows (rare) copy the first computed result
    for r, ns in pos.items():
        for n in ns[1:]:
            o[:, :, n], to[:, :, n], lse[:, :, n] = o[:, :, ns[0]], to[:, :, ns[0]], lse[:, :, ns[0]]
    return o, to, lse

