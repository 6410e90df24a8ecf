"""attn_bwd_noalloc (the gradient entry point that allocates nothing) against
attn_bwd on the same inputs, through the C ABI.

Two calls in a row, the second on a smaller input, then the first again: the
library's per-GPU array for D keeps the previous call's contents, and every
call must still equal attn_bwd (same kernels, so bit for bit) and stay within
the gradient tolerance of the fp64 oracle ("Causal-rCM", Sec. 3.1.1, Eq. 8:
the backward of the packed teacher-forcing attention).
"""
import numpy as np
import pytest
import torch

import attention_jvp_causal_amd as aj
from attention_jvp_causal_amd.workloads import Workload, make_inputs
from oracle import attn_vjp_ref
from parity_util import max_abs, oracle_mask, rel_l2, to_np

pytestmark = pytest.mark.gpu

REL_L2, REL_MAX = 1e-2, 2e-2

CASES = [
    # the larger input first, then a smaller one with another head_dim, then the first again
    Workload("noalloc_a", 2, 3, 128, "bf16", "block_causal", 6, 70, 2, seed=201),
    Workload("noalloc_b", 1, 2, 64, "bf16", "tf_clean_noisy", 3, 50, 1, seed=202),
]


def _grads(w, dev, dO, desc, fn, out_dtype):
    o, lse = aj.attn_fwd(dev["q"], dev["k"], dev["v"], desc, scale=w.scale)
    B, H, L, D = w.shape
    outs = tuple(torch.full((B, H, L, D), float("nan"), dtype=out_dtype, device="cuda") for _ in range(3))
    if fn is aj.attn_bwd:
        delta = torch.full((B, H, L), float("nan"), dtype=torch.float32, device="cuda")
        dq, dk, dv, _ = aj.attn_bwd(dev["q"], dev["k"], dev["v"], o, dO, lse, desc, scale=w.scale,
                                    out_dtype=out_dtype, out=outs + (delta,))
    else:
        dq, dk, dv = aj.attn_bwd_noalloc(dev["q"], dev["k"], dev["v"], o, dO, lse, desc, scale=w.scale,
                                         out_dtype=out_dtype, out=outs)
    torch.cuda.synchronize()
    return dq, dk, dv


def test_noalloc_gradients_equal_attn_bwd_on_consecutive_calls():
    ref_cache = {}
    for step, w in enumerate([CASES[0], CASES[1], CASES[0]]):
        print(f"[case] attn_bwd_noalloc call {step}: {w.name} shape={w.shape}", flush=True)
        inputs = make_inputs(w)
        dev = {n: t.cuda() for n, t in inputs.items()}
        g = torch.Generator().manual_seed(300 + w.seed)
        dO = torch.randn(w.shape, generator=g).to(torch.bfloat16)
        desc = aj.attn_jvp_mask_desc_build(w.mask_kind, w.num_frames, w.frame_tokens, w.frames_per_chunk,
                                           head_dim=w.head_dim, dtype=w.dtype)
        want = _grads(w, dev, dO.cuda(), desc, aj.attn_bwd, torch.float32)
        got = _grads(w, dev, dO.cuda(), desc, aj.attn_bwd_noalloc, torch.float32)
        for name, a, b in zip(("dq", "dk", "dv"), got, want):
            assert torch.equal(a, b), f"{w.name} {name}: attn_bwd_noalloc differs from attn_bwd"
        if w.name not in ref_cache:
            x = {n: t.to(torch.float64).numpy() for n, t in inputs.items()}
            ref_cache[w.name] = attn_vjp_ref(x["q"], x["k"], x["v"], dO.double().numpy(), oracle_mask(w),
                                             scale=w.scale)
        for name, a, r in zip(("dq", "dk", "dv"), got, ref_cache[w.name]):
            a = to_np(a)
            e2, ea = rel_l2(a, r), max_abs(a, r)
            assert e2 <= REL_L2 and ea <= REL_MAX * float(np.abs(r).max()), f"{w.name} {name}: {e2:.2e} {ea:.2e}"
        print(f"[ok] call {step}: equal to attn_bwd bit for bit, within tolerance of the oracle", flush=True)
