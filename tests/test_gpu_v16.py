"""attn_jvp_fwd_v16 (the d = 64 JVP reading fp16 copies of V and tV that a
conversion kernel writes first) against attn_jvp_fwd, which converts every key
tile in the kernel's local memory: the same conversion of the same values, so
O, tO and lse must agree bit for bit.  The copies themselves are checked
against V and tV, and one case against the fp64 oracle ("Causal-rCM", App. B,
Eqs. 42-45).
"""
import pytest
import torch

import attention_jvp_causal_amd as aj
from attention_jvp_causal_amd.workloads import WORKLOADS, Workload, as_float64, make_inputs
from oracle import attn_jvp_ref
from parity_util import compare, oracle_mask, to_np

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "tq", "tk", "tv")


def _desc(w):
    return aj.attn_jvp_mask_desc_build(w.mask_kind, w.num_frames, w.frame_tokens, w.frames_per_chunk,
                                       head_dim=w.head_dim, dtype=w.dtype)


def _check_copies(v, v16):
    # bf16 values of magnitude in [2^-14, 65504] are fp16 values: copied
    # exactly; smaller ones keep fp16's subnormal resolution (2^-24)
    x, y = v.float(), v16.float()
    big = x.abs() >= 2.0 ** -14
    assert torch.equal(x[big], y[big]), "fp16 copy differs on a representable value"
    assert bool(((x - y).abs()[~big] <= 2.0 ** -24).all()), "fp16 copy of a small value off by more than 2^-24"


def _same(w, dev, desc, scale=None, out_dtype=None, label=""):
    scale = w.scale if scale is None else scale
    plain = aj.attn_jvp_fwd(*(dev[n] for n in NAMES), desc, scale=scale, out_dtype=out_dtype)
    v16 = (torch.empty_like(dev["v"], dtype=torch.float16), torch.empty_like(dev["tv"], dtype=torch.float16))
    fast = aj.attn_jvp_fwd_v16(*(dev[n] for n in NAMES), desc, scale=scale, out_dtype=out_dtype, v16=v16)
    torch.cuda.synchronize()
    for name, a, b in zip(("o", "to", "lse"), fast, plain):
        assert torch.equal(a, b), f"{label}: {name} differs from attn_jvp_fwd"
    _check_copies(dev["v"], v16[0])
    _check_copies(dev["tv"], v16[1])
    print(f"[ok] {label}: bitwise equal to attn_jvp_fwd", flush=True)
    return fast


CASES = [
    # name, kind, T, F, c, B, H, sigmas, scale (None: 1/8, folded into Q), out dtype
    ("c3_d64", "block_causal", 6, 88, 3, 1, 3, (1, 1, 1), None, None),
    ("stress_d64_ragged", "block_causal", 7, 61, 3, 2, 2, (3, 1, 0.5), None, None),
    ("stress_d64_f32_out", "block_causal", 6, 88, 3, 2, 2, (3, 1, 0.5), None, torch.float32),
    ("scale_not_pow2", "block_causal", 5, 70, 2, 1, 2, (1, 1, 1), 0.1, None),
    ("full_d64", "full", 2, 150, 1, 1, 2, (1, 1, 1), None, None),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bitwise_equal_to_attn_jvp_fwd(case):
    name, kind, T, F, c, B, H, (sq, sv, st), scale, out_dtype = case
    w = Workload(name, B, H, 64, "bf16", kind, T, F, c, seed=300 + CASES.index(case), sigma_qk=sq, sigma_v=sv,
                 sigma_t=st)
    print(f"[case] {name} B={B} H={H} L={w.seq_len} scale={scale} out={out_dtype}", flush=True)
    dev = {n: t.cuda() for n, t in make_inputs(w).items()}
    _same(w, dev, _desc(w), scale=scale, out_dtype=out_dtype, label=name)


def test_against_the_oracle():
    w = Workload("stress_v16", 2, 2, 64, "bf16", "block_causal", 6, 88, 3, seed=311, sigma_qk=3, sigma_v=1,
                 sigma_t=0.5)
    print(f"[case] {w.name} L={w.seq_len} vs oracle", flush=True)
    inputs = make_inputs(w)
    dev = {n: t.cuda() for n, t in inputs.items()}
    got = aj.attn_jvp_fwd_v16(*(dev[n] for n in NAMES), _desc(w), scale=w.scale)
    torch.cuda.synchronize()
    x = as_float64(inputs)
    ref = attn_jvp_ref(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], oracle_mask(w), scale=w.scale)
    res = compare(w, [to_np(t) for t in got], ref, label=w.name)
    print(f"[ok] {w.name}: " + ", ".join(f"{k} relL2={v[0]:.2e} maxabs={v[1]:.2e}" for k, v in res.items()), flush=True)


def test_strided_layout():
    # [B, L, H, D] storage viewed as [B, H, L, D]: the copies take v's strides
    w = Workload("blhd_v16", 2, 3, 64, "bf16", "block_causal", 5, 64, 1, seed=312)
    print(f"[case] {w.name} [B, L, H, D] storage", flush=True)
    dev = {n: t.permute(0, 2, 1, 3).contiguous().cuda().permute(0, 2, 1, 3) for n, t in make_inputs(w).items()}
    assert dev["v"].stride() != (w.heads * w.seq_len * 64, w.seq_len * 64, 64, 1)
    _same(w, dev, _desc(w), label=w.name)


def test_tangent_free_declaration():
    # teacher forcing with the clean half declared: primal-only tiles through
    # the primal kernel, the rest through the variants instance on the copies
    w = Workload("tf_v16", 1, 2, 64, "bf16", "tf_clean_noisy", 4, 90, 2, seed=313, clean_tangent_zero=True)
    print(f"[case] {w.name} L={w.seq_len} clean half tangent-free", flush=True)
    dev = {n: t.cuda() for n, t in make_inputs(w).items()}
    fast = aj.attn_jvp_mask_desc_tangent_free(_desc(w), [(0, w.seq_len // 2)])
    assert fast.work()[1] > 0 and fast.work()[2] > 0
    _same(w, dev, fast, label=w.name)


@pytest.mark.parametrize("wname", ["stress_chunk3_d64", "tf_clean_noisy_d64"])
def test_full_size_bitwise(wname):
    w = WORKLOADS[wname]
    print(f"[case] full-size {w.name}", flush=True)
    dev = {n: t.cuda() for n, t in make_inputs(w).items()}
    _same(w, dev, _desc(w), label=w.name)


def test_rejected_without_a_launch():
    w = Workload("rej_v16", 1, 1, 128, "bf16", "full", 1, 64, 1, seed=314)
    dev = {n: t.cuda() for n, t in make_inputs(w).items()}
    with pytest.raises(aj.AttnJvpError) as e:
        aj.attn_jvp_fwd_v16(*(dev[n] for n in NAMES), _desc(w))
    assert e.value.status == aj.AJ_ENOTSUP
    w64 = Workload("rej_v16_64", 1, 1, 64, "bf16", "full", 1, 64, 1, seed=315)
    dev = {n: t.cuda() for n, t in make_inputs(w64).items()}
    with pytest.raises(ValueError):
        aj.attn_jvp_fwd_v16(*(dev[n] for n in NAMES), _desc(w64), v16=(dev["v"], dev["tv"]))  # bf16, not fp16
