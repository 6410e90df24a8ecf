"""Frame-level attention masks, written from the pages' descriptions.

Test infrastructure (see the package docstring).  Independent of the C++ mask
descriptor builder: this file states *which* (query, key) pairs are allowed,
token by token, and nothing about tiles.

Source: "Causal-rCM" Sec. 2.3 (causal attention across frames / chunks),
Sec. 3.1.1 and Eq. 8 (teacher forcing packs [clean | noisy]; each noisy block
attends to the clean frames before it that it may use, plus the tokens of its
own noisy block), App. B (a mask is a set of
admissible query-key rectangles), and the reading notes' mask table (full
within a frame, causal across frames; block-causal is full within a chunk and
causal across chunks).

Readings where the pages are silent or disagree (each listed in the design
notes):
* a frame (chunk) sees itself: attention inside a frame is always full;
* teacher forcing: clean chunk i sees clean chunks <= i; noisy chunk i sees
  clean chunks < i and its own noisy chunk (noisy chunk 0 sees only itself);
* a ragged last chunk (num_frames not a multiple of frames_per_chunk) is a
  shorter chunk of the remaining frames.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

import numpy as np

FULL = "full"
BLOCK_CAUSAL = "block_causal"
TF_CLEAN_NOISY = "tf_clean_noisy"


@dataclass(frozen=True)
class MaskLayout:
    kind: str
    num_frames: int
    frame_tokens: int
    frames_per_chunk: int = 1

    @property
    def half_len(self) -> int:
        return self.num_frames * self.frame_tokens

    @property
    def seq_len(self) -> int:
        return 2 * self.half_len if self.kind == TF_CLEAN_NOISY else self.half_len

    def chunk_of(self, tok: int) -> int:
        """Chunk index of a token position inside one [frames x tokens] stream."""
        return (tok // self.frame_tokens) // self.frames_per_chunk

    def chunk_end(self, c: int) -> int:
        """One past the last token of chunk c inside one stream."""
        return min((c + 1) * self.frames_per_chunk * self.frame_tokens, self.half_len)

    def chunk_begin(self, c: int) -> int:
        return c * self.frames_per_chunk * self.frame_tokens


@dataclass(frozen=True)
class RectMask:
    """A mask given directly as admissible rectangles [q0,q1) x [k0,k1) (App. B).

    seq_len is the number of query rows; kv_len the number of keys when the
    keys are another sequence (a query chunk over a KV cache, Sec. 3.2.1
    "KV Cache"), else the same as seq_len."""
    seq_len: int
    rects: Tuple[Tuple[int, int, int, int], ...]
    kv_len: Optional[int] = None

    @property
    def key_len(self) -> int:
        return self.seq_len if self.kv_len is None else self.kv_len


def chunk_over_cache(chunk_len: int, prefix_len: int) -> RectMask:
    """Readonly KV-cache attention of one chunk (Sec. 3.2.1 "KV Cache"): the
    chunk's queries see the committed prefix and, with the chunk's own keys
    placed after it, every key of the chunk (attention inside a chunk is full)."""
    kv = prefix_len + chunk_len
    return RectMask(chunk_len, ((0, chunk_len, 0, kv),), kv_len=kv)


def allowed(mask, i: int, j: int) -> bool:
    """Element predicate: may query token i attend to key token j?"""
    if isinstance(mask, RectMask):
        return any(q0 <= i < q1 and k0 <= j < k1 for (q0, q1, k0, k1) in mask.rects)
    L = mask.seq_len
    if not (0 <= i < L and 0 <= j < L):
        return False
    if mask.kind == FULL:
        return True
    if mask.kind == BLOCK_CAUSAL:
        return mask.chunk_of(j) <= mask.chunk_of(i)
    if mask.kind == TF_CLEAN_NOISY:
        n = mask.half_len
        qi_noisy, kj_noisy = i >= n, j >= n
        ci = mask.chunk_of(i - n if qi_noisy else i)
        cj = mask.chunk_of(j - n if kj_noisy else j)
        if not qi_noisy:                       # clean query: clean history incl. itself
            return (not kj_noisy) and cj <= ci
        if kj_noisy:                           # noisy query: only its own noisy chunk
            return cj == ci
        return cj < ci                         # ... and strictly earlier clean chunks
    raise ValueError(f"unknown mask kind {mask.kind!r}")


def key_ranges(mask, i: int) -> List[Tuple[int, int]]:
    """Allowed keys of query row i as sorted, disjoint half-open ranges."""
    if isinstance(mask, RectMask):
        rs = sorted((k0, k1) for (q0, q1, k0, k1) in mask.rects if q0 <= i < q1 and k0 < k1)
        out: List[Tuple[int, int]] = []
        for a, b in rs:
            if out and a <= out[-1][1]:
                out[-1] = (out[-1][0], max(out[-1][1], b))
            else:
                out.append((a, b))
        return out
    L = mask.seq_len
    if not 0 <= i < L:
        return []
    if mask.kind == FULL:
        return [(0, L)]
    if mask.kind == BLOCK_CAUSAL:
        return [(0, mask.chunk_end(mask.chunk_of(i)))]
    if mask.kind == TF_CLEAN_NOISY:
        n = mask.half_len
        if i < n:
            return [(0, mask.chunk_end(mask.chunk_of(i)))]
        c = mask.chunk_of(i - n)
        own = (n + mask.chunk_begin(c), n + mask.chunk_end(c))
        return [(0, mask.chunk_begin(c)), own] if c > 0 else [own]
    raise ValueError(f"unknown mask kind {mask.kind!r}")


def dense_mask(mask) -> np.ndarray:
    """Boolean [L, Lk] matrix built from the element predicate (tiny L only)."""
    L = mask.seq_len
    Lk = mask.key_len if isinstance(mask, RectMask) else L
    return np.array([[allowed(mask, i, j) for j in range(Lk)] for i in range(L)], dtype=bool)


def unmasked_pairs(mask) -> int:
    """Number of allowed (query, key) pairs, summed over per-row key ranges."""
    return sum(b - a for i in range(mask.seq_len) for (a, b) in key_ranges(mask, i))


def frame_grid(mask) -> np.ndarray:
    """Frame-level picture of a layout: entry [f, g] is 1 when frame f sees frame g.

    Frames are numbered along the packed sequence (clean frames first for TF).
    Used to compare against the hand-written grids under tests/golden/.
    """
    F = mask.frame_tokens
    nf = mask.seq_len // F
    return np.array([[1 if allowed(mask, f * F, g * F) else 0 for g in range(nf)]
                     for f in range(nf)], dtype=np.int64)
