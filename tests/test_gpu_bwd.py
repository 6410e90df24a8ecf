"""HIP gradients of masked attention (attn_bwd) vs the fp64 gradient oracle.

The GPU path runs attn_fwd for O and lse and then attn_bwd; the oracle
computes dq, dk, dv from q, k, v, dO alone.  Tolerance for bf16 operands
(P and dS are rounded to bf16 once, accumulation is fp32): rel-L2 <= 1e-2 per
tensor, as for the forward, and max-abs <= 2e-2 of the tensor's largest
reference magnitude (gradient magnitudes grow with the number of queries that
see a key, so an absolute bound alone would not scale).
"""
import numpy as np
import pytest
import torch

import attention_jvp_causal_amd as aj
from attention_jvp_causal_amd.workloads import WORKLOADS, Workload, make_inputs
from oracle import RectMask, attn_vjp_ref, attn_vjp_sampled, dense_mask
from parity_util import max_abs, oracle_mask, rel_l2, to_np

pytestmark = pytest.mark.gpu

REL_L2, REL_MAX = 1e-2, 2e-2


def _cotangent(w, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(w.shape, generator=g, dtype=torch.float32).to(torch.bfloat16)


def _check(name, got, ref, label):
    got = np.asarray(got, np.float64)
    e2 = rel_l2(got, ref)
    ea = max_abs(got, ref)
    scale = max(1e-30, float(np.abs(ref).max()))
    print(f"[ok] {label} {name} relL2={e2:.2e} maxabs={ea:.2e} (max|ref| {scale:.2e})", flush=True)
    assert e2 <= REL_L2, f"{label} {name}: rel-L2 {e2:.3e}"
    assert ea <= REL_MAX * scale, f"{label} {name}: max-abs {ea:.3e} vs {REL_MAX} x {scale:.3e}"


def _run(w, desc, inputs, dO, out_dtype=None):
    dev = {n: t.cuda() for n, t in inputs.items()}
    o, lse = aj.attn_fwd(dev["q"], dev["k"], dev["v"], desc, scale=w.scale)
    dq, dk, dv, delta = aj.attn_bwd(dev["q"], dev["k"], dev["v"], o, dO.cuda(), lse, desc, scale=w.scale,
                                    out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv, delta


def _layout_desc(w):
    return aj.attn_jvp_mask_desc_build(w.mask_kind, w.num_frames, w.frame_tokens, w.frames_per_chunk,
                                       head_dim=w.head_dim, dtype=w.dtype)


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
def test_reduced_every_element(case):
    kind, T, F, c, B, H, D, odt = case
    w = Workload("bwd", B, H, D, "bf16", kind, T, F, c, seed=80 + CASES.index(case))
    print(f"[case] bwd {kind} T={T} F={F} c={c} B={B} H={H} D={D} out={odt}", flush=True)
    inputs = make_inputs(w)
    dO = _cotangent(w, 90 + CASES.index(case))
    _, _, dq, dk, dv, delta = _run(w, _layout_desc(w), inputs, dO, odt)
    x = {n: t.to(torch.float64).numpy() for n, t in inputs.items()}
    ref = attn_vjp_ref(x["q"], x["k"], x["v"], dO.to(torch.float64).numpy(), oracle_mask(w), scale=w.scale)
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        _check(name, to_np(g), r, kind)
    if odt is not None:
        assert dq.dtype == odt and dk.dtype == odt


def test_rect_mask_with_unused_rows_and_keys():
    L, D = 300, 128
    rects = ((0, 100, 0, 100), (130, 300, 0, 40), (130, 300, 150, 300))  # rows 100..129 see nothing,
    w = Workload("bwd_rects", 2, 2, D, "bf16", "full", 1, L, 1, seed=95)  # keys 100..149 are unseen
    print("[case] bwd rects", flush=True)
    inputs = make_inputs(w)
    dO = _cotangent(w, 96)
    desc = aj.attn_jvp_mask_desc_from_rects(L, rects, head_dim=D, dtype="bf16")
    o, lse, dq, dk, dv, delta = _run(w, desc, inputs, dO, torch.float32)
    assert (dq[:, :, 100:130] == 0).all()
    assert (dk[:, :, 100:150] == 0).all() and (dv[:, :, 100:150] == 0).all()
    x = {n: t.to(torch.float64).numpy() for n, t in inputs.items()}
    ref = attn_vjp_ref(x["q"], x["k"], x["v"], dO.to(torch.float64).numpy(), RectMask(L, rects), scale=w.scale)
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        _check(name, to_np(g), r, "rects")


def test_determinism_and_sum_rules():
    w = Workload("bwd_inv", 1, 2, 128, "bf16", "block_causal", 6, 70, 2, seed=97)
    inputs = make_inputs(w)
    dO = _cotangent(w, 98)
    desc = _layout_desc(w)
    a = _run(w, desc, inputs, dO, torch.float32)
    b = _run(w, desc, inputs, dO, torch.float32)
    for x, y in zip(a, b):
        assert torch.equal(x, y), "reruns must be bitwise identical"
    _, _, dq, dk, dv, _ = a
    # shifting every key by one vector changes nothing: sum_j dK_j = 0
    s = dk.double().sum(dim=2).abs().max().item()
    assert s <= 1e-2 * dk.double().abs().sum(dim=2).max().item()
    # attention weights sum to one: sum_j dV_j = sum_i dO_i
    np.testing.assert_allclose(dv.double().sum(dim=2).cpu().numpy(), dO.double().sum(dim=2).numpy(),
                               rtol=2e-2, atol=2e-2)


@pytest.mark.parametrize("wname", ["wan13b_chunk3_causal", "stress_chunk3_d64"])
def test_full_size_sampled(wname):
    w = WORKLOADS[wname]
    print(f"[case] bwd full-size {wname}", flush=True)
    inputs = make_inputs(w)
    dO = _cotangent(w, 99)
    _, _, dq, dk, dv, delta = _run(w, _layout_desc(w), inputs, dO)
    assert torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()
    L = w.seq_len
    rng = np.random.default_rng(5)
    rows = sorted({0, L - 1, L // 2} | set(int(r) for r in rng.integers(0, L, 12)))
    keys = sorted({0, L - 1, 4679, 4680} | set(int(r) for r in rng.integers(0, L, 12)))
    heads = [(0, 0), (w.batch - 1, w.heads - 1)]
    x = {n: t.to(torch.float64).numpy() for n, t in inputs.items()}
    sq, sk, sv = attn_vjp_sampled(x["q"], x["k"], x["v"], dO.to(torch.float64).numpy(), oracle_mask(w),
                                  rows, keys, heads, scale=w.scale)
    for (b, h) in heads:
        _check("dq", to_np(dq[b, h, rows]), sq[(b, h)], f"{wname} b{b}h{h}")
        _check("dk", to_np(dk[b, h, keys]), sk[(b, h)], f"{wname} b{b}h{h}")
        _check("dv", to_np(dv[b, h, keys]), sv[(b, h)], f"{wname} b{b}h{h}")


@pytest.mark.parametrize("D", [128, 64])
def test_strided_layout(D):
    # inputs stored [B, L, H, D] and viewed as [B, H, L, D] (the five inputs
    # share those strides); outputs in a permuted layout of their own
    w = Workload("bwd_strided", 2, 3, D, "bf16", "block_causal", 4, 75, 2, seed=100 + D)
    print(f"[case] bwd strided D={D}", flush=True)
    inputs = make_inputs(w)
    B, H, L, _ = w.shape
    desc = _layout_desc(w)

    def blhd(t):  # same values, [B, L, H, D] storage
        return t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)

    q, k, v = (blhd(inputs[n]).cuda() for n in ("q", "k", "v"))
    assert q.stride() != inputs["q"].stride()
    o, lse = aj.attn_fwd(q, k, v, desc, scale=w.scale)
    # the forward's default output takes the inputs' layout, so it feeds the
    # gradients as it is
    assert o.stride() == q.stride()
    o_s = o
    dO = _cotangent(w, 101)
    dO_s = blhd(dO).cuda()
    outs = tuple(torch.empty((B, L, H, D), dtype=torch.float32, device="cuda").permute(0, 2, 1, 3)
                 for _ in range(3)) + (torch.empty((B, H, L), dtype=torch.float32, device="cuda"),)
    dq, dk, dv, _ = aj.attn_bwd(q, k, v, o_s, dO_s, lse, desc, scale=w.scale, out_dtype=torch.float32, out=outs)
    torch.cuda.synchronize()
    # the same call on contiguous tensors gives the same bits
    c = {n: inputs[n].cuda() for n in ("q", "k", "v")}
    o_c, lse_c = aj.attn_fwd(c["q"], c["k"], c["v"], desc, scale=w.scale)
    assert torch.equal(o_c, o) and torch.equal(lse_c, lse)
    dq_c, dk_c, dv_c, _ = aj.attn_bwd(c["q"], c["k"], c["v"], o_c, dO.cuda(), lse_c, desc, scale=w.scale,
                                      out_dtype=torch.float32)
    torch.cuda.synchronize()
    for name, a, b in (("dq", dq, dq_c), ("dk", dk, dk_c), ("dv", dv, dv_c)):
        assert torch.equal(a, b), f"strided {name} differs from the contiguous call"
    x = {n: t.to(torch.float64).numpy() for n, t in inputs.items()}
    ref = attn_vjp_ref(x["q"], x["k"], x["v"], dO.to(torch.float64).numpy(), oracle_mask(w), scale=w.scale)
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        _check(name, to_np(g), r, f"strided d{D}")
