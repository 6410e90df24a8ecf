"""Helpers for the GPU parity tests: run the HIP path and the oracle on the
same seeded inputs and compare with the stated tolerances."""
import numpy as np

from attention_jvp_causal_amd.workloads import Workload, make_inputs, as_float64
from oracle import MaskLayout, attn_jvp_ref

# Tolerances for the HIP path against the fp64 oracle:
#  fp32 inputs: rel-L2 <= 1e-5; bf16 inputs: rel-L2 <= 1e-2 and max-abs <= 5e-2.
TOL = {"f32": {"rel_l2": 1e-5, "max_abs": None}, "bf16": {"rel_l2": 1e-2, "max_abs": 5e-2}}


def rel_l2(x, y):
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    den = np.linalg.norm(y)
    return float(np.linalg.norm(x - y) / (den if den > 0 else 1.0))


def max_abs(x, y):
    return float(np.max(np.abs(np.asarray(x, np.float64) - np.asarray(y, np.float64)))) if np.size(y) else 0.0


def lse_gap_bound(D):
    """Largest |lse_fwd - lse_jvp| the two roundings allow.  Each path sums l
    from p~ rounded to bf16 (8 significant bits: relative error up to 2^-8 at
    the bottom of a binade) or, in the d = 64 JVP, to fp16 (up to 2^-11), so
    each ln l is within ln(1 + u) of the exact one; 1e-4 covers the fp32
    arithmetic around it."""
    u_jvp = 2.0 ** -11 if D == 64 else 2.0 ** -8
    return np.log1p(2.0 ** -8) + np.log1p(u_jvp) + 1e-4


def oracle_mask(w: Workload) -> MaskLayout:
    return MaskLayout(w.mask_kind, w.num_frames, w.frame_tokens, w.frames_per_chunk)


def run_gpu(w: Workload, inputs=None, out_dtype=None, device="cuda"):
    import torch
    import attention_jvp_causal_amd as aj

    if inputs is None:
        inputs = make_inputs(w)
    dev = {n: t.to(device) for n, t in inputs.items()}
    desc = aj.attn_jvp_mask_desc_build(w.mask_kind, w.num_frames, w.frame_tokens, w.frames_per_chunk,
                                       head_dim=w.head_dim, dtype=w.dtype)
    o, to, lse = aj.attn_jvp_fwd(dev["q"], dev["k"], dev["v"], dev["tq"], dev["tk"], dev["tv"], desc,
                                 scale=w.scale, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return inputs, desc, (o, to, lse)


def to_np(t):
    import torch

    return t.detach().to("cpu", torch.float64).numpy()


def compare(w: Workload, got, ref, label=""):
    """Returns a dict of errors and asserts the tolerances for O, tO and lse."""
    tol = TOL[w.dtype]
    res = {}
    for name, g, r in zip(("o", "to", "lse"), got, ref):
        finite = np.isfinite(r)
        assert np.array_equal(np.isfinite(g), finite), f"{label} {name}: non-finite pattern differs"
        gg, rr = g[finite], r[finite]
        res[name] = (rel_l2(gg, rr), max_abs(gg, rr))
        assert res[name][0] <= tol["rel_l2"], f"{label} {name}: rel-L2 {res[name][0]:.3e} > {tol['rel_l2']}"
        if tol["max_abs"] is not None:
            assert res[name][1] <= tol["max_abs"], f"{label} {name}: max-abs {res[name][1]:.3e} > {tol['max_abs']}"
    return res


def sample_rows(w: Workload, n_random=40, seed=0):
    """Rows at every frame edge, query-tile edges near frames, the ragged end,
    plus random rows."""
    L, F = w.seq_len, w.frame_tokens
    rows = {0, L - 1}
    for f in range(L // F):
        rows |= {f * F, f * F + F - 1}
    for qt in (1, (L // 128) // 2, L // 128 - 1):
        rows |= {qt * 128 - 1, qt * 128}
    rng = np.random.default_rng(seed)
    rows |= set(int(x) for x in rng.integers(0, L, size=n_random))
    return sorted(r for r in rows if 0 <= r < L)


class WholeTensorErrors:
    """Accumulates rel-L2 (over the whole tensor) and max-abs (over every
    element) of O, tO and lse while the oracle runs one (batch, head) at a
    time, so that full-size workloads fit in host memory."""

    NAMES = ("o", "to", "lse")

    def __init__(self, w: Workload, label=""):
        self.w, self.label = w, label
        self.err2 = dict.fromkeys(self.NAMES, 0.0)
        self.ref2 = dict.fromkeys(self.NAMES, 0.0)
        self.amax = dict.fromkeys(self.NAMES, 0.0)
        self.where = dict.fromkeys(self.NAMES, None)
        self.count = dict.fromkeys(self.NAMES, 0)

    def add(self, got, ref, bh):
        for name, g, r in zip(self.NAMES, got, ref):
            finite = np.isfinite(r)
            assert np.array_equal(np.isfinite(g), finite), f"{self.label} {name} bh={bh}: non-finite pattern differs"
            d = np.abs(np.asarray(g, np.float64)[finite] - r[finite])
            self.err2[name] += float(np.dot(d, d))
            self.ref2[name] += float(np.dot(r[finite], r[finite]))
            self.count[name] += int(d.size)
            if d.size and d.max() > self.amax[name]:
                self.amax[name] = float(d.max())
                self.where[name] = (bh, int(np.argmax(np.where(finite, np.abs(np.asarray(g, np.float64) - r), -1))))

    def result(self):
        return {n: (float(np.sqrt(self.err2[n] / self.ref2[n])) if self.ref2[n] > 0 else float(np.sqrt(self.err2[n])),
                    self.amax[n]) for n in self.NAMES}

    def check(self):
        tol = TOL[self.w.dtype]
        res = self.result()
        for n, (rl2, ma) in res.items():
            assert rl2 <= tol["rel_l2"], f"{self.label} {n}: rel-L2 {rl2:.3e} > {tol['rel_l2']}"
            if tol["max_abs"] is not None:
                assert ma <= tol["max_abs"], (f"{self.label} {n}: max-abs {ma:.3e} > {tol['max_abs']} "
                                              f"at (bh, flat index) {self.where[n]}")
        return res
