"""Edge cases of the HIP path at the size and structure extremes.

* a sequence of 2^18 tokens, checked on sampled rows against the oracle;
* a batch stride of 2^31 elements (element offsets beyond 32 bits) for the
  inputs and the outputs;
* a mask that allows nothing (every row: O = tO = 0, lse = -inf);
* many (batch, head) pairs with a tiny sequence (grid dominated by B x H);
* a single token.
"""
import numpy as np
import pytest
import torch

import attention_jvp_causal_amd as aj
from attention_jvp_causal_amd.workloads import Workload, as_float64, make_inputs
from oracle import RectMask, attn_jvp_ref
from parity_util import compare, oracle_mask, run_gpu, to_np

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "tq", "tk", "tv")


def test_longest_sequence_sampled_rows():
    # 2^18 tokens = 16 frames x 16384, chunks of 4 frames: ~2.1e10 pairs per head
    w = Workload("long", 1, 2, 128, "bf16", "block_causal", 16, 16384, 4, seed=150)
    print(f"[case] long L={w.seq_len}", flush=True)
    inputs, desc, (o, to, lse) = run_gpu(w)
    assert torch.isfinite(o).all() and torch.isfinite(to).all() and torch.isfinite(lse).all()
    L = w.seq_len
    rows = [0, 1, 65535, 65536, 131071, 131072, 200000, L - 129, L - 128, L - 1]
    x = {n: t.to(torch.float64).numpy() for n, t in inputs.items()}
    ref = attn_jvp_ref(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], oracle_mask(w), scale=w.scale, rows=rows)
    res = compare(w, [to_np(o[:, :, rows]), to_np(to[:, :, rows]), to_np(lse[:, :, rows])], ref, label="long")
    print("[ok] long: " + ", ".join(f"{k} relL2={v[0]:.2e} maxabs={v[1]:.2e}" for k, v in res.items()), flush=True)


def test_offsets_beyond_32_bits():
    # B = 2 with a batch stride of 2^31 elements: batch 1 starts 4 GiB into
    # each buffer.  The six inputs share one buffer (same strides), as do O, tO.
    B, H, L, D = 2, 2, 300, 128
    w = Workload("far", B, H, D, "bf16", "block_causal", 3, 100, 1, seed=154)
    inputs = make_inputs(w)
    n = H * L * D
    sb = 1 << 31
    print(f"[case] far: batch stride {sb} elements", flush=True)
    buf = torch.zeros(sb + 6 * n, dtype=torch.bfloat16, device="cuda")
    views = {}
    for t, name in enumerate(NAMES):
        v = torch.as_strided(buf, (B, H, L, D), (sb, L * D, D, 1), storage_offset=t * n)
        v.copy_(inputs[name].cuda())
        views[name] = v
    obuf = torch.zeros(sb + 2 * n, dtype=torch.bfloat16, device="cuda")
    o = torch.as_strided(obuf, (B, H, L, D), (sb, L * D, D, 1), storage_offset=0)
    to = torch.as_strided(obuf, (B, H, L, D), (sb, L * D, D, 1), storage_offset=n)
    lse = torch.empty((B, H, L), dtype=torch.float32, device="cuda")
    desc = aj.attn_jvp_mask_desc_build("block_causal", 3, 100, 1, head_dim=D, dtype="bf16")
    aj.attn_jvp_fwd(*(views[nm] for nm in NAMES), desc, out=(o, to, lse))
    torch.cuda.synchronize()
    x = as_float64(inputs)
    ref = attn_jvp_ref(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], oracle_mask(w), scale=w.scale)
    compare(w, [to_np(o), to_np(to), to_np(lse)], ref, label="far")
    del buf, obuf


@pytest.mark.parametrize("D", [128, 64])
def test_mask_that_allows_nothing(D):
    L = 200
    w = Workload("empty", 1, 2, D, "bf16", "full", 1, L, 1, seed=151)
    dev = {n: t.cuda() for n, t in make_inputs(w).items()}
    desc = aj.attn_jvp_mask_desc_from_rects(L, [], head_dim=D, dtype="bf16")
    assert desc.unmasked_pairs == 0
    o, to, lse = aj.attn_jvp_fwd(*(dev[n] for n in NAMES), desc)
    o2, lse2 = aj.attn_fwd(dev["q"], dev["k"], dev["v"], desc)
    torch.cuda.synchronize()
    assert (o == 0).all() and (to == 0).all() and torch.isneginf(lse).all()
    assert (o2 == 0).all() and torch.isneginf(lse2).all()


def test_many_heads_tiny_sequence():
    w = Workload("manyheads", 8, 64, 64, "bf16", "block_causal", 3, 11, 1, seed=152)
    print(f"[case] many heads B={w.batch} H={w.heads} L={w.seq_len}", flush=True)
    inputs, desc, got = run_gpu(w)
    x = as_float64(inputs)
    ref = attn_jvp_ref(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], oracle_mask(w), scale=w.scale)
    compare(w, [to_np(t) for t in got], ref, label="manyheads")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_single_token(dt):
    w = Workload("one", 1, 3, 128, dt, "full", 1, 1, 1, seed=153)
    inputs, desc, got = run_gpu(w)
    x = as_float64(inputs)
    ref = attn_jvp_ref(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], oracle_mask(w), scale=w.scale)
    compare(w, [to_np(t) for t in got], ref, label=f"one_{dt}")
    # one key: O = v, tO = tv exactly up to output rounding
    np.testing.assert_allclose(to_np(got[0]), x["v"], rtol=1e-2, atol=1e-2)
    np.testing.assert_allclose(to_np(got[1]), x["tv"], rtol=1e-2, atol=1e-2)


@pytest.mark.parametrize("D", [128, 64])
def test_head_groups_with_a_ragged_last_group(D):
    # Workgroups are taken eight heads at a time; B x H = 21 leaves a last
    # group of 5 heads, and 3 query tiles per head make several ranks per head.
    w = Workload("hgroups", 3, 7, D, "bf16", "block_causal", 3, 100, 1, seed=155)
    print(f"[case] head groups B={w.batch} H={w.heads} L={w.seq_len} D={D}", flush=True)
    inputs, desc, got = run_gpu(w)
    x = as_float64(inputs)
    ref = attn_jvp_ref(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], oracle_mask(w), scale=w.scale)
    compare(w, [to_np(t) for t in got], ref, label=f"hgroups_{D}")
    # the primal forward and the gradients walk the same grid order
    from oracle import attn_vjp_ref

    dev = {n: t.cuda() for n, t in inputs.items()}
    o, lse = aj.attn_fwd(dev["q"], dev["k"], dev["v"], desc, scale=w.scale)
    g = torch.Generator().manual_seed(156)
    d_out = torch.randn(w.shape, generator=g).to(torch.bfloat16)
    dq, dk, dv, _ = aj.attn_bwd(dev["q"], dev["k"], dev["v"], o, d_out.cuda(), lse, desc, scale=w.scale)
    torch.cuda.synchronize()
    np.testing.assert_allclose(to_np(lse), ref[2], rtol=0, atol=1e-2)
    gref = attn_vjp_ref(x["q"], x["k"], x["v"], d_out.double().numpy(), oracle_mask(w), scale=w.scale)
    for name, t, r in zip(("dq", "dk", "dv"), (dq, dk, dv), gref):
        t = to_np(t)
        err = np.linalg.norm(t - r) / np.linalg.norm(r)
        assert err <= 1e-2, f"hgroups_{D} {name}: rel-L2 {err:.3e}"


def test_binding_rejects_outputs_on_another_device():
    # the C ABI sees plain pointers; the binding checks that preallocated
    # outputs live on the inputs' device before passing them on
    w = Workload("dev", 1, 1, 64, "bf16", "full", 1, 64, 1, seed=157)
    dev = {n: t.cuda() for n, t in make_inputs(w).items()}
    desc = aj.attn_jvp_mask_desc_build("full", 1, 64, 1, head_dim=64, dtype="bf16")
    host = (torch.empty(w.shape, dtype=torch.bfloat16), torch.empty(w.shape, dtype=torch.bfloat16),
            torch.empty((1, 1, 64), dtype=torch.float32))
    with pytest.raises(ValueError):
        aj.attn_jvp_fwd(*(dev[n] for n in NAMES), desc, out=host)
    with pytest.raises(ValueError):
        aj.attn_fwd(dev["q"], dev["k"], dev["v"], desc, out=(host[0], host[2]))
    kvd = aj.attn_jvp_mask_desc_from_rects_kv(64, 64, [(0, 64, 0, 64)], head_dim=64, dtype="bf16")
    with pytest.raises(ValueError):
        aj.attn_fwd_kv(dev["q"], dev["k"], dev["v"], kvd, out=(host[0], host[2]))
