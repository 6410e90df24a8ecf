"""HIP JVP with tangent-free token ranges (the clean-context fast path) vs the
fp64 oracle and vs the same call without the declaration.

When the declared tangents are zero, the skipped products only ever add exact
zeros.  Query tiles that keep some tangent work run the JVP kernel's variant
instance: their O and lse are bitwise those of the plain descriptor's run.
Query tiles left with only primal work run the primal forward kernel (tO = 0
written): equal to rounding, as for attn_fwd (at d = 128 32-row instead of
16-row waves, at d = 64 p~ in bf16 instead of the JVP's fp16).  tO is equal in value everywhere; against the oracle the usual
tolerances apply.
"""
import numpy as np
import pytest
import torch

import attention_jvp_causal_amd as aj
from attention_jvp_causal_amd.workloads import WORKLOADS, Workload, as_float64, make_inputs
from oracle import RectMask, attn_jvp_ref
from parity_util import compare, lse_gap_bound, oracle_mask, sample_rows, to_np

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "tq", "tk", "tv")


def _run(dev, desc, out_dtype=None):
    r = aj.attn_jvp_fwd(*(dev[n] for n in NAMES), desc, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return r


def _primal_rows(desc):
    """Rows of the query tiles whose visited tiles are all tangent-free (read
    from the descriptor's tile variants)."""
    L, tm, tn = desc.seq_len, 128, 64
    n_kt = (desc.kv_len + tn - 1) // tn
    rows = torch.zeros(L, dtype=torch.bool)
    for qt in range((L + tm - 1) // tm):
        if all(desc.tile_variant(qt, kt) in (-1, 3) for kt in range(n_kt)):
            rows[qt * tm:(qt + 1) * tm] = True
    return rows


def _same_as_plain(fast, plain, label, desc):
    # equal in value (a zero may differ in sign)
    assert bool((fast[1] == plain[1]).all()), f"{label}: tO differs from the plain descriptor's"
    pr = _primal_rows(desc).to(fast[0].device)
    jr = ~pr
    assert torch.equal(fast[0][:, :, jr], plain[0][:, :, jr]), f"{label}: O differs on the JVP rows"
    assert torch.equal(fast[2][:, :, jr], plain[2][:, :, jr]), f"{label}: lse differs on the JVP rows"
    if not bool(pr.any()):
        return
    o, o_p = fast[0][:, :, pr], plain[0][:, :, pr]
    lse, lse_p = fast[2][:, :, pr], plain[2][:, :, pr]
    do = (o.float() - o_p.float()).abs().max().item()
    dl = (lse - lse_p).abs().max().item()
    print(f"[cmp] {label} primal rows: max|dO| {do:.2e} max|dlse| {dl:.2e}", flush=True)
    assert do <= 2e-2 * max(1.0, o_p.float().abs().max().item()), f"{label}: O on the primal rows"
    assert dl <= lse_gap_bound(desc.head_dim), f"{label}: lse on the primal rows"


def _layout_desc(w):
    return aj.attn_jvp_mask_desc_build(w.mask_kind, w.num_frames, w.frame_tokens, w.frames_per_chunk,
                                       head_dim=w.head_dim, dtype=w.dtype)


@pytest.mark.parametrize("D,out_dtype", [(128, None), (128, torch.float32), (64, None)])
def test_teacher_forcing_reduced_every_element(D, out_dtype):
    w = Workload(f"tf_fast_d{D}", 1, 2, D, "bf16", "tf_clean_noisy", 4, 90, 1, seed=41, clean_tangent_zero=True)
    print(f"[case] {w.name} L={w.seq_len} out={out_dtype}", flush=True)
    inputs = make_inputs(w)
    dev = {n: t.cuda() for n, t in inputs.items()}
    base = _layout_desc(w)
    fast = aj.attn_jvp_mask_desc_tangent_free(base, [(0, w.seq_len // 2)])
    assert fast.work()[2] > 0 and fast.work()[1] > 0
    got = _run(dev, fast, out_dtype)
    _same_as_plain(got, _run(dev, base, out_dtype), w.name, fast)
    x = as_float64(inputs)
    ref = attn_jvp_ref(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], oracle_mask(w), scale=w.scale)
    res = compare(w, [to_np(t) for t in got], ref, label=w.name)
    assert (got[1][:, :, : w.seq_len // 2] == 0).all()
    print(f"[ok] {w.name}: " + ", ".join(f"{k} relL2={v[0]:.2e} maxabs={v[1]:.2e}" for k, v in res.items()),
          flush=True)


RECT_CASES = [
    # L, rects, tangent-free ranges, D
    (420, ((0, 200, 0, 200), (200, 420, 0, 130), (200, 420, 200, 420)), [(0, 200)], 128),
    (420, ((0, 200, 0, 200), (200, 420, 0, 130), (200, 420, 200, 420)), [(0, 128), (300, 333)], 128),
    (333, ((0, 333, 0, 333),), [(64, 192), (256, 333)], 128),
    (333, ((0, 100, 0, 50), (100, 333, 40, 333)), [(0, 256)], 64),
]


@pytest.mark.parametrize("case", RECT_CASES, ids=[f"rect{i}" for i in range(len(RECT_CASES))])
def test_rect_masks_with_tangent_free_ranges(case):
    L, rects, ranges, D = case
    w = Workload("rect_tf", 2, 2, D, "bf16", "full", 1, L, 1, seed=43 + RECT_CASES.index(case))
    print(f"[case] rects L={L} D={D} ranges={ranges}", flush=True)
    inputs = make_inputs(w)
    for a, b in ranges:  # the declaration must hold: zero tangents there
        for n in ("tq", "tk", "tv"):
            inputs[n][:, :, a:b] = 0
    dev = {n: t.cuda() for n, t in inputs.items()}
    base = aj.attn_jvp_mask_desc_from_rects(L, rects, head_dim=D, dtype="bf16")
    fast = aj.attn_jvp_mask_desc_tangent_free(base, ranges)
    got = _run(dev, fast)
    _same_as_plain(got, _run(dev, base), "rects", fast)
    x = as_float64(inputs)
    ref = attn_jvp_ref(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], RectMask(L, rects), scale=w.scale)
    compare(w, [to_np(t) for t in got], ref, label="rects")


@pytest.mark.parametrize("wname", ["wan13b_tf_clean_noisy", "tf_clean_noisy_d64"])
def test_full_size_teacher_forcing_fast_path(wname):
    w = WORKLOADS[wname]
    print(f"[case] full-size {w.name} with the clean half tangent-free", flush=True)
    inputs = make_inputs(w)
    dev = {n: t.cuda() for n, t in inputs.items()}
    base = _layout_desc(w)
    fast = aj.attn_jvp_mask_desc_tangent_free(base, [(0, w.seq_len // 2)])
    assert fast.work()[1] > 0, "keys-tangent-free tiles present"
    got = _run(dev, fast)
    plain = _run(dev, base)
    _same_as_plain(got, plain, w.name, fast)
    del plain
    o, to, lse = got
    assert (to[:, :, : w.seq_len // 2] == 0).all()
    rows = sample_rows(w)
    x = {n: t.to(torch.float64).numpy() for n, t in inputs.items()}
    ref = attn_jvp_ref(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], oracle_mask(w), scale=w.scale, rows=rows)
    res = compare(w, [to_np(o[:, :, rows]), to_np(to[:, :, rows]), to_np(lse[:, :, rows])], ref, label=w.name)
    print(f"[ok] {w.name} fast rows={len(rows)}: " + ", ".join(f"{k} relL2={v[0]:.2e} maxabs={v[1]:.2e}"
                                                              for k, v in res.items()), flush=True)
