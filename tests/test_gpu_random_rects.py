"""JVP, primal forward and gradients on seeded random rectangle masks (App. B:
a mask is any set of admissible query-key rectangles) vs the fp64 oracles.

Each case cuts the queries into bands of random height and gives every band
a few disjoint key intervals of random position and width, so tile edges,
partial tiles, rows with no allowed key and keys no query sees all occur at
sizes that span several 128 x 64 tiles.
"""
import numpy as np
import pytest
import torch

import attention_jvp_causal_amd as aj
from attention_jvp_causal_amd.workloads import Workload, as_float64, make_inputs
from oracle import RectMask, attn_jvp_ref, attn_vjp_ref
from parity_util import compare, rel_l2, to_np

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "tq", "tk", "tv")


def random_rects(L, rng):
    """Disjoint rectangles: query bands, each with up to three disjoint key intervals."""
    rects, q = [], 0
    while q < L:
        h = int(rng.integers(1, 160))
        q1 = min(L, q + h)
        if rng.random() < 0.1:  # a band that sees nothing
            q = q1
            continue
        cuts = sorted(set(int(x) for x in rng.integers(0, L + 1, size=6)))
        pairs = [(cuts[i], cuts[i + 1]) for i in range(0, len(cuts) - 1, 2)][:3]
        for k0, k1 in pairs:
            if k0 < k1:
                rects.append((q, q1, k0, k1))
        q = q1
    return rects


CASES = [(seed, D, L) for seed, (D, L) in enumerate([(128, 450), (64, 333), (128, 700), (64, 512), (128, 257), (64, 641)])]


@pytest.mark.parametrize("seed,D,L", CASES, ids=[f"s{s}_d{d}_L{l}" for s, d, l in CASES])
def test_random_rectangles(seed, D, L):
    rng = np.random.default_rng(1000 + seed)
    rects = random_rects(L, rng)
    print(f"[case] random rects seed={seed} D={D} L={L} n={len(rects)}", flush=True)
    w = Workload(f"rand{seed}", 1, 2, D, "bf16", "full", 1, L, 1, seed=200 + seed)
    inputs = make_inputs(w)
    dev = {n: t.cuda() for n, t in inputs.items()}
    desc = aj.attn_jvp_mask_desc_from_rects(L, rects, head_dim=D, dtype="bf16")
    mask = RectMask(L, tuple(rects))
    x = as_float64(inputs)

    o, to, lse = aj.attn_jvp_fwd(*(dev[n] for n in NAMES), desc, scale=w.scale)
    torch.cuda.synchronize()
    ref = attn_jvp_ref(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], mask, scale=w.scale)
    compare(w, [to_np(o), to_np(to), to_np(lse)], ref, label=f"rand{seed} jvp")

    o_f, lse_f = aj.attn_fwd(dev["q"], dev["k"], dev["v"], desc, scale=w.scale)
    torch.cuda.synchronize()
    compare(w, [to_np(o_f), np.zeros_like(ref[1]), to_np(lse_f)], (ref[0], np.zeros_like(ref[1]), ref[2]),
            label=f"rand{seed} fwd")

    g = torch.Generator().manual_seed(300 + seed)
    d_out = torch.randn(w.shape, generator=g).to(torch.bfloat16)
    dq, dk, dv, _ = aj.attn_bwd(dev["q"], dev["k"], dev["v"], o_f, d_out.cuda(), lse_f, desc, scale=w.scale,
                                out_dtype=torch.float32)
    torch.cuda.synchronize()
    gref = attn_vjp_ref(x["q"], x["k"], x["v"], d_out.double().numpy(), mask, scale=w.scale)
    for name, t, r in zip(("dq", "dk", "dv"), (dq, dk, dv), gref):
        t = to_np(t)
        assert np.isfinite(t).all(), f"rand{seed} {name}: non-finite values"
        if np.abs(r).max() == 0:
            assert np.abs(t).max() == 0, f"rand{seed} {name}: nonzero where the gradient is zero"
            continue
        err = rel_l2(t, r)
        print(f"[ok] rand{seed} {name} relL2={err:.2e}", flush=True)
        assert err <= 1e-2, f"rand{seed} {name}: rel-L2 {err:.3e}"
        assert np.abs(t - r).max() <= 2e-2 * np.abs(r).max(), f"rand{seed} {name}: max-abs"
