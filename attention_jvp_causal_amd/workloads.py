"""Seeded synthetic workloads for the custom-mask attention JVP.

This module holds the workload shapes and the input generator shared by the
HIP path's tests/bench and by the fp64 oracle.  It contains none of the
method's arithmetic: it only draws random numbers and lays them out.

Shapes follow the Wan2.1 480p latent geometry described in "Causal-rCM: A
Unified Teacher-Forcing and Self-Forcing Open Recipe for Autoregressive
Diffusion Distillation" (Sec. 5 setup: 81 RGB frames -> 21 latent frames) and
the reading notes' worked token example (a 104x60 latent with 2x2 patches gives
30x52 = 1560 tokens per frame).  Chunking c3-3 (3 frames per chunk) and the
teacher-forcing [clean | noisy] packing come from Sec. 3.1.1 (Eq. 8) of the
paper.  The inputs are i.i.d. Gaussians, the plainest stand-in for activations
whose distribution the pages do not give.

Recipe: ``numpy.random.default_rng(seed)`` (PCG64); draw
``standard_normal(dtype=float32) * sigma`` in the order q, k, v, tq, tk, tv,
each of shape [B, H, L, d]; cast to the workload dtype with round-to-nearest-
even (torch).  The oracle receives the same rounded values upcast exactly to
float64.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Tuple

import numpy as np

# Mask layout kinds, spelled the same way on both sides of the C ABI.
MASK_FULL = "full"
MASK_BLOCK_CAUSAL = "block_causal"      # chunks of c frames; c = 1 is frame-causal
MASK_TF_CLEAN_NOISY = "tf_clean_noisy"  # [clean | noisy] teacher-forcing packing


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    head_dim: int
    dtype: str               # "f32" or "bf16"
    mask_kind: str
    num_frames: int          # frames (per half for the TF layout)
    frame_tokens: int
    frames_per_chunk: int
    seed: int
    sigma_qk: float = 1.0
    sigma_v: float = 1.0
    sigma_t: float = 1.0
    clean_tangent_zero: bool = False   # TF layout: tangents are 0 on clean tokens
    notes: str = ""

    @property
    def seq_len(self) -> int:
        n = self.num_frames * self.frame_tokens
        return 2 * n if self.mask_kind == MASK_TF_CLEAN_NOISY else n

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))

    @property
    def shape(self) -> Tuple[int, int, int, int]:
        return (self.batch, self.heads, self.seq_len, self.head_dim)

    def mask_tuple(self):
        return (self.mask_kind, self.num_frames, self.frame_tokens, self.frames_per_chunk)


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny_frame_causal_f32", 1, 2, 64, "f32", MASK_BLOCK_CAUSAL, 4, 16, 1, seed=1,
                 notes="4 frames x 16 tokens, frame-causal, fp32"),
        Workload("wan13b_frame_causal", 1, 12, 128, "bf16", MASK_BLOCK_CAUSAL, 21, 1560, 1, seed=2,
                 notes="Wan2.1-1.3B-shaped, 21 x 1560 tokens, frame-causal (c1-1)"),
        Workload("wan13b_chunk3_causal", 1, 12, 128, "bf16", MASK_BLOCK_CAUSAL, 21, 1560, 3, seed=3,
                 notes="Wan2.1-1.3B-shaped, 7 chunks of 3 frames x 1560 tokens, block-causal (c3-3)"),
        Workload("wan13b_tf_clean_noisy", 1, 12, 128, "bf16", MASK_TF_CLEAN_NOISY, 21, 1560, 1, seed=4,
                 clean_tangent_zero=True,
                 notes="Teacher-forcing [21 clean | 21 noisy] frames x 1560 tokens"),
        Workload("stress_chunk3_d64", 2, 24, 64, "bf16", MASK_BLOCK_CAUSAL, 21, 880, 3, seed=5,
                 sigma_qk=3.0, sigma_v=1.0, sigma_t=0.5,
                 notes="online-softmax stress: large logits, 7 chunks x 3 x 880 tokens, d=64"),
        # One GPU's share under head-parallel (Ulysses) sequence sharding over 4
        # GPUs: 3 of the 12 heads at the full sequence length.
        Workload("wan13b_chunk3_causal_h3", 1, 3, 128, "bf16", MASK_BLOCK_CAUSAL, 21, 1560, 3, seed=6,
                 notes="c3-3 at 3 heads: one GPU's share of the 12 heads over 4 GPUs"),
        Workload("wan13b_tf_clean_noisy_h3", 1, 3, 128, "bf16", MASK_TF_CLEAN_NOISY, 21, 1560, 1, seed=7,
                 clean_tangent_zero=True,
                 notes="teacher forcing at 3 heads: one GPU's share of the 12 heads over 4 GPUs"),
        # Teacher forcing at head_dim 64, for the tangent-free fast path of the
        # 32-row kernel: the stress workload's head count and frame size.
        Workload("tf_clean_noisy_d64", 2, 24, 64, "bf16", MASK_TF_CLEAN_NOISY, 21, 880, 3, seed=8,
                 clean_tangent_zero=True,
                 notes="teacher forcing c3-3 [21 clean | 21 noisy] frames x 880 tokens, d=64"),
    ]
}

# Order in which the workloads are listed (small correctness case first).
WORKLOAD_ORDER = list(WORKLOADS)
BENCH_WORKLOAD = "wan13b_chunk3_causal"


def with_shape(w: Workload, **kw) -> Workload:
    """A copy of ``w`` with some fields replaced (used for reduced-size tests)."""
    d = {f: getattr(w, f) for f in w.__dataclass_fields__}
    d.update(kw)
    return Workload(**d)


def draw_inputs_f32(w: Workload) -> Dict[str, np.ndarray]:
    """Draw q, k, v, tq, tk, tv as float32 arrays of shape [B, H, L, d]."""
    rng = np.random.default_rng(w.seed)
    sig = {"q": w.sigma_qk, "k": w.sigma_qk, "v": w.sigma_v,
           "tq": w.sigma_t, "tk": w.sigma_t, "tv": w.sigma_t}
    out = {}
    for name in ("q", "k", "v", "tq", "tk", "tv"):
        a = rng.standard_normal(size=w.shape, dtype=np.float32)
        if sig[name] != 1.0:
            a *= np.float32(sig[name])
        out[name] = a
    if w.clean_tangent_zero:
        half = w.seq_len // 2
        for name in ("tq", "tk", "tv"):
            out[name][:, :, :half, :] = 0.0
    return out


def make_inputs(w: Workload):
    """Inputs as CPU torch tensors in the workload dtype (RNE cast for bf16)."""
    import torch

    tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    arrs = draw_inputs_f32(w)
    return {n: torch.from_numpy(a).to(tdt) for n, a in arrs.items()}


def as_float64(tensors) -> Dict[str, np.ndarray]:
    """Exact fp64 copies of the (possibly bf16) input tensors, for the oracle."""
    import torch

    return {n: t.to(torch.float64).numpy() for n, t in tensors.items()}
