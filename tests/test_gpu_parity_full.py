"""The full-size workloads against the fp64 oracle on every element.

For each measured workload the HIP path runs once in the launch configuration
bench.py times (bf16 outputs) and once with fp32 outputs; the oracle then runs
one (batch, head) at a time and both results are compared with it on every
element of O, tO and lse: rel-L2 over the whole tensor and max-abs over every
element, at the bf16 tolerances ("Causal-rCM", App. B, Eqs. 42-45: the primal
output and its tangent in the online form).  The fp32-output run separates the
kernel's own arithmetic error from the final rounding of the outputs to bf16.
"""
import time

import numpy as np
import pytest
import torch

from attention_jvp_causal_amd.workloads import WORKLOADS
from oracle import attn_jvp_ref
from parity_util import WholeTensorErrors, oracle_mask, run_gpu, to_np

pytestmark = pytest.mark.gpu

FULL = ["wan13b_frame_causal", "wan13b_chunk3_causal", "wan13b_tf_clean_noisy", "stress_chunk3_d64"]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wname", FULL)
def test_full_size_workload_every_element(wname):
    w = WORKLOADS[wname]
    B, H, L, D = w.shape
    print(f"[case] whole-tensor {wname} shape={w.shape} {w.dtype}", flush=True)
    inputs, _, got = run_gpu(w)
    _, _, got32 = run_gpu(w, inputs=inputs, out_dtype=torch.float32)
    o, to, lse = got
    assert torch.isfinite(o).all() and torch.isfinite(to).all() and torch.isfinite(lse).all()
    if w.clean_tangent_zero:
        assert (to[:, :, :L // 2] == 0).all(), "clean rows must have exactly zero tangent"
    host = [t.cpu() for t in got]
    host32 = [t.cpu() for t in got32]
    del got, got32
    torch.cuda.empty_cache()
    acc = WholeTensorErrors(w, label=f"{wname} bf16-out")
    acc32 = WholeTensorErrors(w, label=f"{wname} f32-out")
    mask = oracle_mask(w)
    t0 = time.perf_counter()
    for bh in range(B * H):
        b, h = divmod(bh, H)
        x = {n: t[b:b + 1, h:h + 1].to(torch.float64).numpy() for n, t in inputs.items()}
        ref = attn_jvp_ref(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], mask, scale=w.scale)
        acc.add([to_np(t[b:b + 1, h:h + 1]) for t in host], ref, bh)
        acc32.add([to_np(t[b:b + 1, h:h + 1]) for t in host32], ref, bh)
        if bh % 4 == 3 or bh == B * H - 1:
            print(f"  {wname}: {bh + 1}/{B * H} heads, {time.perf_counter() - t0:.0f} s", flush=True)
    for a in (acc32, acc):
        res = a.result()
        print(f"[result] {a.label}: " + ", ".join(f"{k} relL2={v[0]:.2e} maxabs={v[1]:.2e}" for k, v in res.items()),
              flush=True)
    acc32.check()
    acc.check()
