"""The gradients at full size against the fp64 oracle on every element.

attn_fwd then attn_bwd run once on the two workloads bench.py times for the
gradients (the c3-3 Wan2.1 shape at head_dim 128 and the d = 64 stress
workload), in that launch configuration (bf16 outputs); the gradient oracle
then runs one (batch, head) at a time and every element of dq, dk and dv is
compared: rel-L2 over the whole tensor <= 1e-2 and max-abs <= 2e-2 of the
tensor's largest reference magnitude, the gradient tolerance of the other
gradient tests (the chain rule of "Causal-rCM" App. B, Eq. 42, taken through
the packed teacher-forcing forward of Sec. 3.1.1, Eq. 8).
"""
import time

import numpy as np
import pytest
import torch

import attention_jvp_causal_amd as aj
from attention_jvp_causal_amd.workloads import WORKLOADS, make_inputs
from oracle import attn_vjp_ref
from parity_util import oracle_mask

pytestmark = pytest.mark.gpu

REL_L2, REL_MAX = 1e-2, 2e-2


class _Acc:
    """Whole-tensor error sums of one gradient, gathered head by head."""

    def __init__(self):
        self.err2 = self.ref2 = self.max_err = self.max_ref = 0.0

    def add(self, got, ref):
        d = got - ref
        self.err2 += float((d * d).sum())
        self.ref2 += float((ref * ref).sum())
        self.max_err = max(self.max_err, float(np.abs(d).max()))
        self.max_ref = max(self.max_ref, float(np.abs(ref).max()))

    def rel_l2(self):
        return (self.err2 / self.ref2) ** 0.5 if self.ref2 > 0 else self.err2 ** 0.5


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wname", ["wan13b_chunk3_causal", "stress_chunk3_d64"])
def test_full_size_gradients_every_element(wname):
    w = WORKLOADS[wname]
    B, H, L, D = w.shape
    print(f"[case] whole-tensor gradients {wname} shape={w.shape}", flush=True)
    inputs = make_inputs(w)
    g = torch.Generator().manual_seed(123)
    dO = torch.randn(w.shape, generator=g, dtype=torch.float32).to(torch.bfloat16)
    desc = aj.attn_jvp_mask_desc_build(w.mask_kind, w.num_frames, w.frame_tokens, w.frames_per_chunk,
                                       head_dim=D, dtype=w.dtype)
    dev = {n: inputs[n].cuda() for n in ("q", "k", "v")}
    o, lse = aj.attn_fwd(dev["q"], dev["k"], dev["v"], desc, scale=w.scale)
    dq, dk, dv, _ = aj.attn_bwd(dev["q"], dev["k"], dev["v"], o, dO.cuda(), lse, desc, scale=w.scale)
    torch.cuda.synchronize()
    got = {n: t.cpu() for n, t in (("dq", dq), ("dk", dk), ("dv", dv))}
    for n, t in got.items():
        assert t.dtype == torch.bfloat16 and torch.isfinite(t).all(), n
    del dev, o, lse, dq, dk, dv
    torch.cuda.empty_cache()
    acc = {n: _Acc() for n in got}
    mask = oracle_mask(w)
    t0 = time.perf_counter()
    for bh in range(B * H):
        b, h = divmod(bh, H)
        x = {n: inputs[n][b:b + 1, h:h + 1].to(torch.float64).numpy() for n in ("q", "k", "v")}
        ref = attn_vjp_ref(x["q"], x["k"], x["v"], dO[b:b + 1, h:h + 1].to(torch.float64).numpy(), mask,
                           scale=w.scale)
        for n, r in zip(("dq", "dk", "dv"), ref):
            acc[n].add(got[n][b:b + 1, h:h + 1].to(torch.float64).numpy(), r)
        if bh % 4 == 3 or bh == B * H - 1:
            print(f"  {wname}: {bh + 1}/{B * H} heads, {time.perf_counter() - t0:.0f} s", flush=True)
    for n, a in acc.items():
        print(f"[result] {wname} {n}: relL2={a.rel_l2():.2e} maxabs={a.max_err:.2e} (max|ref| {a.max_ref:.2e})",
              flush=True)
    for n, a in acc.items():
        assert a.rel_l2() <= REL_L2, f"{wname} {n}: rel-L2 {a.rel_l2():.3e}"
        assert a.max_err <= REL_MAX * a.max_ref, f"{wname} {n}: max-abs {a.max_err:.3e} vs {REL_MAX} x {a.max_ref:.3e}"
