"""fp64 CPU oracle for the custom-mask attention JVP.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything here.  The
product path (the HIP kernels behind the C ABI and their Python binding) never
imports this package, and this package imports nothing from the product.

What it computes follows "Causal-rCM: A Unified Teacher-Forcing and
Self-Forcing Open Recipe for Autoregressive Diffusion Distillation", App. B
("FlashAttention-2 JVP Kernel with Custom Masks"): masked softmax attention
(Eq. 42), its score tangent (Eq. 43), zero tangent on masked-out entries, and
the attention tangent written as sums over valid keys (Eq. 44).  The mask
layouts follow Sec. 2.3 / Sec. 3.1.1 (teacher forcing, Eq. 8) and the chunk
patterns c1-1 / c3-3 of Sec. 5.

Pins (tests/test_oracle.py, tests/test_oracle_masks.py, tests/test_oracle_kv.py):
central finite differences of the oracle's own primal, forward-mode autodiff of a dense masked attention,
PyTorch's scaled_dot_product_attention and scipy's logsumexp as library special
cases, per-element brute force on tiny inputs, the invariants of the JVP
(linearity, zero tangents, tQ = tK = 0, masked-key perturbation, constant
values, shift invariance), closed-form pair counts and hand-written frame-level
mask grids.  The gradients (tests/test_oracle_vjp.py) are pinned by reverse-mode
autodiff of a dense masked attention and of PyTorch's SDPA, by the adjoint
identity with the (separately pinned) JVP, by central finite differences and by
their sum rules.  Every function here is pinned; none is "parity unpinned".
"""
from .masks import MaskLayout, RectMask, allowed, chunk_over_cache, key_ranges, dense_mask, unmasked_pairs
from .attention_jvp import attn_jvp_ref
from .attention_vjp import attn_vjp_ref, attn_vjp_sampled

__all__ = [
    "MaskLayout", "RectMask", "allowed", "chunk_over_cache", "key_ranges", "dense_mask", "unmasked_pairs",
    "attn_jvp_ref", "attn_vjp_ref", "attn_vjp_sampled",
]
