"""HIP query-chunk-over-KV-cache forward (attn_fwd_kv) vs the fp64 oracle.

The keys and values sit in cache buffers longer than the used prefix, with
their own strides; the queries are a separate tensor.  Compared element by
element with the oracle's rectangular mask, and with the rows of the same
chunk in a block-causal forward of the whole sequence (to rounding: the
kernels see the same pairs in a different tile position).
"""
import numpy as np
import pytest
import torch

import attention_jvp_causal_amd as aj
from attention_jvp_causal_amd.workloads import Workload, make_inputs
from oracle import MaskLayout, attn_jvp_ref, chunk_over_cache
from parity_util import TOL, max_abs, rel_l2, to_np

pytestmark = pytest.mark.gpu


def _check(w, got, ref, label):
    tol = TOL["bf16"]
    for name, g, r in zip(("o", "lse"), got, ref):
        e2, ea = rel_l2(g, r), max_abs(g, r)
        print(f"[ok] {label} {name} relL2={e2:.2e} maxabs={ea:.2e}", flush=True)
        assert e2 <= tol["rel_l2"] and ea <= tol["max_abs"], f"{label} {name}: {e2:.3e} / {ea:.3e}"


CASES = [
    # frames T, tokens F, frames per chunk c, chunk index n, B, H, D, cache capacity extra, out dtype
    (6, 70, 2, 2, 1, 2, 128, 37, None),
    (7, 61, 3, 2, 2, 1, 128, 0, torch.float32),
    (5, 90, 1, 4, 1, 2, 64, 100, None),
    (6, 88, 3, 1, 1, 3, 64, 8, torch.float32),
    (4, 33, 1, 0, 1, 1, 128, 5, None),   # first chunk: no prefix
]


@pytest.mark.parametrize("case", CASES, ids=[f"kv{i}" for i in range(len(CASES))])
def test_chunk_over_cache_every_element(case):
    T, F, c, n, B, H, D, extra, odt = case
    w = Workload("kv", B, H, D, "bf16", "block_causal", T, F, c, seed=120 + CASES.index(case))
    print(f"[case] kv T={T} F={F} c={c} chunk={n} B={B} H={H} D={D} extra={extra} out={odt}", flush=True)
    x = make_inputs(w)
    L, C = w.seq_len, c * F
    r0, r1 = n * C, min(L, (n + 1) * C)
    kv = r1
    # cache buffers [B, H, L + extra, D]; the chunk's own keys already in place
    cap = L + extra
    kc = torch.zeros((B, H, cap, D), dtype=torch.bfloat16)
    vc = torch.zeros_like(kc)
    kc[:, :, :L] = x["k"]
    vc[:, :, :L] = x["v"]
    q = x["q"][:, :, r0:r1].contiguous().cuda()
    kc, vc = kc.cuda(), vc.cuda()
    desc = aj.attn_jvp_mask_desc_from_rects_kv(r1 - r0, kv, [(0, r1 - r0, 0, kv)], head_dim=D, dtype="bf16")
    o, lse = aj.attn_fwd_kv(q, kc, vc, desc, out_dtype=odt)
    torch.cuda.synchronize()
    xd = {k: t.to(torch.float64).numpy() for k, t in x.items()}
    z = np.zeros_like(xd["q"])
    ref = attn_jvp_ref(xd["q"][:, :, r0:r1], xd["k"][:, :, :kv], xd["v"][:, :, :kv], z[:, :, r0:r1],
                       z[:, :, :kv], z[:, :, :kv], chunk_over_cache(r1 - r0, r0), scale=w.scale)
    _check(w, [to_np(o), to_np(lse)], [ref[0], ref[2]], "kv")
    # the same rows of the block-causal forward over the whole sequence
    full = aj.attn_jvp_mask_desc_build("block_causal", T, F, c, head_dim=D, dtype="bf16")
    dev = {k: t.cuda() for k, t in x.items()}
    o_f, lse_f = aj.attn_fwd(dev["q"], dev["k"], dev["v"], full, out_dtype=odt)
    torch.cuda.synchronize()
    assert (o.float() - o_f[:, :, r0:r1].float()).abs().max().item() <= 2e-2
    assert (lse - lse_f[:, :, r0:r1]).abs().max().item() <= 4e-3


def test_square_entry_points_reject_a_kv_descriptor():
    w = Workload("kvrej", 1, 1, 128, "bf16", "full", 1, 100, 1, seed=3)
    dev = {k: t.cuda() for k, t in make_inputs(w).items()}
    desc = aj.attn_jvp_mask_desc_from_rects_kv(100, 160, [(0, 100, 0, 160)], head_dim=128, dtype="bf16")
    with pytest.raises(aj.AttnJvpError) as e:
        aj.attn_fwd(dev["q"], dev["k"], dev["v"], desc)
    assert e.value.status == aj.AJ_EMASK
    with pytest.raises(aj.AttnJvpError) as e:
        aj.attn_jvp_fwd(*(dev[n] for n in ("q", "k", "v", "tq", "tk", "tv")), desc)
    assert e.value.status == aj.AJ_EMASK


def test_full_size_last_chunk_of_the_c3_rollout():
    # Wan2.1 shape: chunk 7 of 7 (3 frames x 1560 tokens) over a 6-chunk cache
    T, F, c = 21, 1560, 3
    w = Workload("kv_full", 1, 12, 128, "bf16", "block_causal", T, F, c, seed=3)
    print("[case] kv full-size last chunk", flush=True)
    x = make_inputs(w)
    L, C = w.seq_len, c * F
    r0, r1 = L - C, L
    q = x["q"][:, :, r0:r1].contiguous().cuda()
    kc, vc = x["k"].cuda(), x["v"].cuda()
    desc = aj.attn_jvp_mask_desc_from_rects_kv(C, L, [(0, C, 0, L)], head_dim=128, dtype="bf16")
    o, lse = aj.attn_fwd_kv(q, kc, vc, desc)
    torch.cuda.synchronize()
    rng = np.random.default_rng(2)
    rows = sorted({0, C - 1, 127, 128} | set(int(r) for r in rng.integers(0, C, 16)))
    xd = {k: t.to(torch.float64).numpy() for k, t in x.items()}
    z = np.zeros_like(xd["q"])
    ref = attn_jvp_ref(xd["q"][:, :, r0:r1], xd["k"], xd["v"], z[:, :, r0:r1], z, z, chunk_over_cache(C, r0),
                       scale=w.scale, rows=rows)
    _check(w, [to_np(o[:, :, rows]), to_np(lse[:, :, rows])], [ref[0], ref[2]], "kv_full")
