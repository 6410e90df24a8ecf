"""HIP primal masked attention (attn_fwd) vs the fp64 oracle and vs the JVP.

attn_fwd rounds p~ to bf16 for its value products; the JVP kernels do so at
head_dim 128 (16-row waves, a different summation order) and round it to fp16
at 64.  Either way O and lse agree with the JVP's to rounding.  Against the
oracle's O and lse the usual bf16 tolerances apply.
"""
import numpy as np
import pytest
import torch

import attention_jvp_causal_amd as aj
from attention_jvp_causal_amd.workloads import WORKLOADS, Workload, as_float64, make_inputs
from oracle import attn_jvp_ref
from parity_util import TOL, lse_gap_bound, max_abs, oracle_mask, rel_l2, sample_rows, to_np

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "tq", "tk", "tv")


def _desc(w):
    return aj.attn_jvp_mask_desc_build(w.mask_kind, w.num_frames, w.frame_tokens, w.frames_per_chunk,
                                       head_dim=w.head_dim, dtype=w.dtype)


def _same_as_jvp(o, lse, o_j, lse_j, D):
    # both round p~ (bf16, or fp16 in the d = 64 JVP) before summing l, each
    # against its own running max: lse agrees to the rounding of l, O to a few
    # bf16 units
    do = (o.float() - o_j.float()).abs().max().item()
    dl = (lse - lse_j).abs().max().item()
    print(f"[cmp] d{D} primal vs jvp: max|dO| {do:.2e} max|dlse| {dl:.2e} (bound {lse_gap_bound(D):.2e})", flush=True)
    assert do <= 2e-2 * max(1.0, o_j.float().abs().max().item())
    assert dl <= lse_gap_bound(D)


def _check_primal(w, got, ref, label):
    tol = TOL[w.dtype]
    for name, g, r in zip(("o", "lse"), got, ref):
        finite = np.isfinite(r)
        assert np.array_equal(np.isfinite(g), finite), f"{label} {name}: non-finite pattern differs"
        e2, ea = rel_l2(g[finite], r[finite]), max_abs(g[finite], r[finite])
        print(f"[ok] {label} {name} relL2={e2:.2e} maxabs={ea:.2e}", flush=True)
        assert e2 <= tol["rel_l2"] and ea <= tol["max_abs"], f"{label} {name}: {e2:.3e} / {ea:.3e}"


CASES = [
    # kind, T, F, c, B, H, D, out dtype
    ("block_causal", 5, 100, 1, 1, 2, 128, None),
    ("block_causal", 7, 61, 3, 2, 1, 128, torch.float32),
    ("tf_clean_noisy", 4, 90, 1, 1, 2, 128, None),
    ("block_causal", 6, 88, 3, 1, 3, 64, None),
    ("full", 3, 150, 1, 1, 2, 64, torch.float32),
    ("block_causal", 3, 7, 1, 1, 1, 128, None),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}_d{c[6]}_{i}" for i, c in enumerate(CASES)])
def test_reduced_every_element_and_equal_to_jvp(case):
    kind, T, F, c, B, H, D, odt = case
    w = Workload("primal", B, H, D, "bf16", kind, T, F, c, seed=60 + CASES.index(case))
    print(f"[case] primal {kind} T={T} F={F} c={c} B={B} H={H} D={D} out={odt}", flush=True)
    inputs = make_inputs(w)
    dev = {n: t.cuda() for n, t in inputs.items()}
    desc = _desc(w)
    o, lse = aj.attn_fwd(dev["q"], dev["k"], dev["v"], desc, out_dtype=odt)
    o_j, _, lse_j = aj.attn_jvp_fwd(*(dev[n] for n in NAMES), desc, out_dtype=odt)
    torch.cuda.synchronize()
    _same_as_jvp(o, lse, o_j, lse_j, D)
    x = as_float64(inputs)
    ref = attn_jvp_ref(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], oracle_mask(w), scale=w.scale)
    _check_primal(w, [to_np(o), to_np(lse)], [ref[0], ref[2]], "primal")


@pytest.mark.parametrize("wname", ["wan13b_chunk3_causal", "stress_chunk3_d64"])
def test_full_size_sampled_rows_and_equal_to_jvp(wname):
    w = WORKLOADS[wname]
    print(f"[case] primal full-size {wname}", flush=True)
    inputs = make_inputs(w)
    dev = {n: t.cuda() for n, t in inputs.items()}
    desc = _desc(w)
    o, lse = aj.attn_fwd(dev["q"], dev["k"], dev["v"], desc)
    o_j, _, lse_j = aj.attn_jvp_fwd(*(dev[n] for n in NAMES), desc)
    torch.cuda.synchronize()
    _same_as_jvp(o, lse, o_j, lse_j, w.head_dim)
    rows = sample_rows(w)
    x = {n: t.to(torch.float64).numpy() for n, t in inputs.items()}
    ref = attn_jvp_ref(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], oracle_mask(w), scale=w.scale, rows=rows)
    _check_primal(w, [to_np(o[:, :, rows]), to_np(lse[:, :, rows])], [ref[0], ref[2]], wname)


def test_fp32_inputs_not_supported():
    w = Workload("primal_f32", 1, 1, 64, "f32", "full", 1, 70, 1, seed=3)
    dev = {n: t.cuda() for n, t in make_inputs(w).items()}
    desc = _desc(w)
    with pytest.raises(aj.AttnJvpError) as e:
        aj.attn_fwd(dev["q"], dev["k"], dev["v"], desc)
    assert e.value.status == aj.AJ_ENOTSUP
