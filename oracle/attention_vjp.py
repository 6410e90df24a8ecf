"""fp64 oracle: gradients of masked softmax attention (reverse mode).

Test infrastructure (see the package docstring).

Training through the packed teacher-forcing forward ("Causal-rCM", Sec. 3.1.1,
Eq. 8: the student's loss is taken on the noisy half of one masked attention
pass) needs the gradients of masked attention with respect to Q, K and V.  The
pages do not write them out; they are the chain rule applied to Eq. 42 (a
reading, recorded with the others).  Per (batch, head), with cotangent dO, c
the softmax scale and A(i) the keys query i may attend to:

* P_ij = softmax over j in A(i) of s_ij = c <q_i, k_j>;  O_i = sum_j P_ij v_j
* dv_j  = sum_i P_ij dO_i
* dP_ij = <dO_i, v_j>;  D_i = <dO_i, O_i>;  dS_ij = P_ij (dP_ij - D_i)
* dq_i  = c sum_j dS_ij k_j;  dk_j = c sum_i dS_ij q_i

Pairs outside the mask take no part.  Rows with no allowed key contribute
nothing.  Evaluated densely per query group (rows sharing one allowed-key set)
with numpy fp64 matrix products: no tiles, no online softmax.
"""
from __future__ import annotations

from typing import Iterable, Optional, Sequence

import numpy as np

from .attention_jvp import _ROW_BLOCK, _row_groups
from .masks import key_ranges


def _key_index(ranges) -> np.ndarray:
    return np.concatenate([np.arange(a, b) for a, b in ranges]) if ranges else np.zeros(0, dtype=np.int64)


def attn_vjp_ref(q, k, v, do, mask, scale: Optional[float] = None):
    """(dq, dk, dv) of masked attention for the cotangent do, float64.

    q, k, v, do: arrays [B, H, L, d].  mask: ``MaskLayout`` or ``RectMask``.
    """
    q, k, v, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, do))
    B, H, L, d = q.shape
    c = 1.0 / np.sqrt(d) if scale is None else float(scale)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for grp, ranges in _row_groups(mask, range(L)):
        idx = _key_index(ranges)
        if idx.size == 0:
            continue
        for b_ in range(B):
            for h in range(H):
                K, V = k[b_, h, idx], v[b_, h, idx]
                for r0 in range(0, len(grp), _ROW_BLOCK):
                    blk = grp[r0:r0 + _ROW_BLOCK]
                    Q, dO = q[b_, h, blk], do[b_, h, blk]
                    s = c * (Q @ K.T)
                    e = np.exp(s - s.max(axis=1, keepdims=True))
                    P = e / e.sum(axis=1, keepdims=True)
                    O = P @ V
                    D = (dO * O).sum(axis=1, keepdims=True)
                    dS = P * (dO @ V.T - D)
                    dq[b_, h, blk] = c * (dS @ K)
                    dk[b_, h, idx] += c * (dS.T @ Q)
                    dv[b_, h, idx] += P.T @ dO
    return dq, dk, dv


def attn_vjp_sampled(q, k, v, do, mask, rows: Sequence[int], keys: Sequence[int], heads: Iterable,
                     scale: Optional[float] = None):
    """dq at ``rows`` and dk, dv at ``keys`` for the (b, h) pairs in ``heads``,
    float64, by the same definition as ``attn_vjp_ref``.

    Returns dicts {(b, h): array} of shapes [len(rows), d] and [len(keys), d].
    dk and dv sum over every query that may attend the sampled keys, so each
    such query's softmax is evaluated over its whole allowed-key set.
    """
    q, k, v, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, do))
    B, H, L, d = q.shape
    c = 1.0 / np.sqrt(d) if scale is None else float(scale)
    rows = [int(r) for r in rows]
    keys = np.asarray([int(j) for j in keys])
    out_dq, out_dk, out_dv = {}, {}, {}
    for (b_, h) in heads:
        dq = np.zeros((len(rows), d))
        dk = np.zeros((len(keys), d))
        dv = np.zeros((len(keys), d))
        row_pos = {}
        for n, r in enumerate(rows):
            row_pos.setdefault(r, []).append(n)
        for grp, ranges in _row_groups(mask, range(L)):
            idx = _key_index(ranges)
            if idx.size == 0:
                continue
            sel = np.nonzero(np.isin(keys, idx))[0]        # sampled keys this group sees
            want_rows = [r for r in grp if r in row_pos]
            if sel.size == 0 and not want_rows:
                continue
            K, V = k[b_, h, idx], v[b_, h, idx]
            where = {int(j): n for n, j in enumerate(idx)}
            cols = np.asarray([where[int(keys[s])] for s in sel], dtype=np.int64)
            members = grp if sel.size else want_rows
            for r0 in range(0, len(members), _ROW_BLOCK):
                blk = members[r0:r0 + _ROW_BLOCK]
                Q, dO = q[b_, h, blk], do[b_, h, blk]
                s = c * (Q @ K.T)
                e = np.exp(s - s.max(axis=1, keepdims=True))
                P = e / e.sum(axis=1, keepdims=True)
                D = (dO * (P @ V)).sum(axis=1, keepdims=True)
                dS = P * (dO @ V.T - D)
                if sel.size:
                    dk[sel] += c * (dS[:, cols].T @ Q)
                    dv[sel] += P[:, cols].T @ dO
                for n_blk, r in enumerate(blk):
                    for n in row_pos.get(r, ()):
                        dq[n] = c * (dS[n_blk] @ K)
        out_dq[(b_, h)], out_dk[(b_, h)], out_dv[(b_, h)] = dq, dk, dv
    return out_dq, out_dk, out_dv
