"""Benchmark of the custom-mask attention-JVP forward on one MI355X.

One step = one attn_jvp_fwd launch over the whole workload (all heads and
rows): scores, score tangents, online softmax, the three value products and the
epilogue.  Inputs are seeded synthetic tensors already resident in HBM.

Metric: TFLOP/s of unmasked work, counting 12*d FLOP per allowed
(batch, head, query, key) pair (QK^T 2d, tQK^T + QtK^T 4d, P V 2d, P tV 2d,
(P.tS) V 2d), as a fraction of the MI355X dense bf16 MFMA peak.

Other measurements of the same kernels (one JSON line each, same schema):
  --tangent-free   teacher-forcing workload with the clean half declared
                   tangent-free: `value` stays in the 12d convention (the work
                   of the plain JVP), the roofline counts the FLOPs executed
                   (12d / 8d / 4d per pair by tile class);
  --op fwd         primal masked attention (O, lse): 4d FLOP per pair;
  --op bwd         its gradients (dq, dk, dv from o, lse, dO): 10d FLOP per pair
                   by the usual count of five products (the kernels execute 14d:
                   the scores and dP are formed once per kernel);
  --op kv          rollout step with a KV cache: the workload's last chunk of
                   queries over the whole sequence's keys held as a cache
                   (block-causal workloads): 4d FLOP per pair.

At head_dim 64 the JVP step is attn_jvp_fwd_v16 (a conversion kernel writes
fp16 copies of V and tV into buffers allocated before the timed steps, then
the JVP kernel reads them; same results as attn_jvp_fwd, bit for bit);
--no-v16 times attn_jvp_fwd instead.

Prints one JSON line.  `--gpus N` with N > 1 exits: this build runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X dense bf16 MFMA peak: 256 CUs x 4096 FLOP/clk/CU x 2.4 GHz.
PEAK_BF16_TFLOPS = 2516.6
PEAK_F32_MFMA_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
METRIC = "masked attention-JVP TFLOP/s (unmasked FLOPs) and % of bf16 MFMA peak, 1 GPU"
METRIC_FWD = "masked attention forward TFLOP/s (unmasked FLOPs, 4d per pair) and % of bf16 MFMA peak, 1 GPU"
METRIC_BWD = "masked attention backward TFLOP/s (unmasked FLOPs, 10d per pair) and % of bf16 MFMA peak, 1 GPU"
METRIC_KV = "KV-cache chunk attention TFLOP/s (unmasked FLOPs, 4d per pair) and % of bf16 MFMA peak, 1 GPU"
def kernel_isa_sha(kernel: str):
    """Hash of a kernel instance's generated code, as the build recorded it
    (attention_jvp_causal_amd/libattnjvp.isa.json); kernel is the name
    kernel_name() returns.  None when the build wrote no entry for it."""
    from attention_jvp_causal_amd import build as _build

    if not os.path.exists(_build.ISA_PATH):
        return None
    with open(_build.ISA_PATH) as f:
        isa = json.load(f)
    return isa.get(f"void aj::{kernel}(aj::FwdArgs)") or isa.get(f"void aj::{kernel}(aj::BwdArgs)")


def uses_v16(dtype: str, head_dim: int, op: str = "jvp") -> bool:
    """Whether bench.py runs the JVP through attn_jvp_fwd_v16 (fp16 copies of V
    and tV made by a conversion kernel before the JVP kernel): the bf16 JVP at
    head_dim 64, unless --no-v16."""
    return op == "jvp" and dtype == "bf16" and head_dim == 64


def kernel_name(dtype: str, head_dim: int, out_f32: bool, op: str = "jvp", tangent_free: bool = False,
                scale: float = None, v16: bool = False) -> str:
    """Name of the kernel instance(s) the library launches for this call, in
    launch order; the last one is the kernel the roofline and the traffic
    record describe."""
    b = lambda x: "true" if x else "false"
    o = b(out_f32)
    if op == "bwd":
        dkdv = f"attn_bwd_dkdv32_kernel<64, {o}>" if head_dim == 64 else f"attn_bwd_dkdv_kernel<{head_dim}, {o}>"
        return f"attn_bwd_dq32_kernel<{head_dim}, {o}> + {dkdv}"
    if dtype == "f32":
        return f"attn_jvp_fwd_f32_kernel<{head_dim}>"
    # the last two template arguments: the workgroup's wave count (the primal
    # forward at d = 128 runs 8-wave (256-row) tasks, the primal-only tiles of
    # a tangent-free JVP and every other q32 instance 4-wave (128-row) ones),
    # and whether V and tV come as fp16 copies
    primal = f"attn_jvp_fwd_bf16_q32_kernel<{head_dim}, {o}, false, false, false, 4, false>"
    if op in ("fwd", "kv"):
        return primal if head_dim == 64 else f"attn_jvp_fwd_bf16_q32_kernel<128, {o}, false, false, false, 8, false>"
    if head_dim == 128:
        jvp = f"attn_jvp_fwd_bf16_q16_kernel<128, {o}, {b(tangent_free)}>"
    else:
        s = 1.0 / math.sqrt(head_dim) if scale is None else scale
        m, _ = math.frexp(s)
        jvp = (f"attn_jvp_fwd_bf16_q32_kernel<64, {o}, true, {b(0.0 < s <= 1.0 and m == 0.5)}, {b(tangent_free)}, 4, "
               f"{b(v16)}>")
        if v16:
            jvp = f"bf16_to_f16_kv_kernel<64> + {jvp}"
    # a tangent-free descriptor runs its primal-only query tiles through the
    # primal kernel first
    return f"{primal} + {jvp}" if tangent_free else jvp


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from the rocprofv3 counter runs
    recorded under profiles/, or None if they were taken on another kernel or
    on other code than the kernel the current build holds."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel") != kernel:
        return None
    isa = kernel_isa_sha(rec.get("kernel", ""))
    if isa is None or rec.get("kernel_isa") != isa:
        return None
    return rec.get("bytes_per_launch")


def record_traffic(workload: str, fetch_csv: str, write_csv: str, calib_mib: int, command: str) -> dict:
    """Builds profiles/traffic_<workload>.json from two rocprofv3 --pmc runs
    (FETCH_SIZE, then WRITE_SIZE) of this script with --calib-copy-mib.

    Both counters are in KiB per dispatch.  Each is scaled by the factor that
    makes the device copy of known size read (write) exactly its size, and the
    kernel's dispatches are averaged."""
    import csv
    from collections import defaultdict

    from attention_jvp_causal_amd.workloads import WORKLOADS

    w = WORKLOADS[workload]
    kname = kernel_name(w.dtype, w.head_dim, False, scale=w.scale,
                        v16=uses_v16(w.dtype, w.head_dim)).split(" + ")[-1]
    kname_sym = kname.split("<")[0]

    def per_dispatch(path, counter):
        acc = defaultdict(float)
        names = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    acc[r["Dispatch_Id"]] += float(r["Counter_Value"])
                    names[r["Dispatch_Id"]] = r["Kernel_Name"]
        copy = [v for d, v in acc.items() if "copyBuffer" in names[d]]
        kern = [v for d, v in acc.items() if kname_sym in names[d]]
        if len(copy) != 1 or not kern:
            raise SystemExit(f"{path}: expected one copy dispatch and >=1 {kname_sym} dispatch")
        return copy[0], sum(kern) / len(kern), len(kern)

    calib = calib_mib * (1 << 20)
    fc, fk, nf = per_dispatch(fetch_csv, "FETCH_SIZE")
    wc, wk, nw = per_dispatch(write_csv, "WRITE_SIZE")
    ff, wf = calib / (fc * 1024), calib / (wc * 1024)
    rec = {
        "workload": workload,
        "kernel": kname,
        "kernel_isa": kernel_isa_sha(kname),
        "fetch_size_kib_per_dispatch": round(fk, 1),
        "write_size_kib_per_dispatch": round(wk, 1),
        "dispatches_averaged": [nf, nw],
        "copy_calibration": {"bytes": calib, "fetch_size_kib": fc, "write_size_kib": wc,
                             "fetch_factor": round(ff, 4), "write_factor": round(wf, 4)},
        "bytes_per_launch": int(round(fk * 1024 * ff + wk * 1024 * wf)),
        "command": command,
    }
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    return rec


class ClockSampler:
    """Samples the GPU's current shader clock (the starred level of
    pp_dpm_sclk) and board power (hwmon power1_input or power1_average) from
    sysfs on a thread while the step repeats.  Read-only; the first DRM card
    that exposes the clock is taken (one GPU per process here).  Under the MFMA
    load of these kernels the chip runs below its 2.4 GHz peak, by an amount
    that differs between boards: the clock explains most of the spread of
    results across machines."""

    def __init__(self, period_s: float = 0.02):
        import glob

        self.period = period_s
        self.sclk = self.power = None
        for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
            if os.path.exists(dev + "/pp_dpm_sclk"):
                self.sclk = dev + "/pp_dpm_sclk"
                pw = sorted(glob.glob(dev + "/hwmon/hwmon*/power1_input") +
                            glob.glob(dev + "/hwmon/hwmon*/power1_average"))
                self.power = pw[0] if pw else None
                break
        self.samples = []
        self._stop = threading.Event()
        self._thread = None

    def _read(self):
        mhz = watts = None
        try:
            for line in open(self.sclk).read().splitlines():
                if line.rstrip().endswith("*"):
                    mhz = int(line.split(":")[1].strip().lower().split("mhz")[0])
        except (OSError, ValueError, IndexError):
            pass
        try:
            if self.power:
                watts = int(open(self.power).read()) / 1e6
        except (OSError, ValueError):
            pass
        return mhz, watts

    def _run(self):
        while not self._stop.is_set():
            self.samples.append(self._read())
            self._stop.wait(self.period)

    def start(self):
        if self.sclk:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()

    def stop(self):
        if not self._thread:
            return None
        self._stop.set()
        self._thread.join()
        med = lambda v: sorted(v)[len(v) // 2] if v else None
        mhz = [m for m, _ in self.samples if m is not None]
        watts = [w for _, w in self.samples if w is not None]
        return {"sclk_mhz_median": med(mhz), "sclk_mhz_min": min(mhz) if mhz else None,
                "board_power_w_median": med(watts), "samples": len(self.samples),
                "source": "sysfs pp_dpm_sclk and hwmon power, sampled every 20 ms while the step repeats "
                          "after the timed region"}


def avg_ms_of(ev) -> float:
    return sum(e0.elapsed_time(e1) for e0, e1 in ev) / len(ev)


def cpu_baseline(w, inputs, heads: int):
    """Times the fp64 oracle (as it stands) on the first `heads` heads of batch 0."""
    import numpy as np

    from oracle import MaskLayout, attn_jvp_ref, unmasked_pairs

    try:
        from threadpoolctl import threadpool_info

        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
        blas = ",".join(sorted({p.get("internal_api", "?") for p in threadpool_info()}))
    except Exception:  # pragma: no cover - reporting only
        threads, blas = os.cpu_count(), "unknown"
    m = MaskLayout(w.mask_kind, w.num_frames, w.frame_tokens, w.frames_per_chunk)
    import torch

    x = {n: t[:1, :heads].to(torch.float64).numpy() for n, t in inputs.items()}
    t0 = time.perf_counter()
    attn_jvp_ref(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], m, scale=w.scale)
    dt = time.perf_counter() - t0
    flop = 12.0 * w.head_dim * unmasked_pairs(m) * heads
    return {"value": round(flop / dt / 1e12, 5), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"fp64 numpy oracle ({blas}), batch 0, {heads} of {w.heads} heads, all {w.seq_len} rows; "
                      f"{dt:.1f} s for {flop:.3e} FLOP",
            "seconds": round(dt, 2),
            "affinity_cores": len(os.sched_getaffinity(0))}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None, help="workload name (default: the c3-3 Wan2.1-1.3B shape)")
    ap.add_argument("--out-dtype", default=None, choices=[None, "bf16", "f32"])
    ap.add_argument("--cpu-heads", type=int, default=2, help="heads timed for the oracle baseline (0 = skip)")
    ap.add_argument("--op", default="jvp", choices=["jvp", "fwd", "bwd", "kv"],
                    help="jvp: O, tO, lse (the metric); fwd: primal O, lse only; bwd: dq, dk, dv; "
                         "kv: last chunk over a KV cache")
    ap.add_argument("--no-v16", action="store_true",
                    help="JVP at head_dim 64: call attn_jvp_fwd (fp16 conversion per key tile in LDS) instead of "
                         "attn_jvp_fwd_v16 (fp16 copies of V and tV made once by a conversion kernel)")
    ap.add_argument("--tangent-free", action="store_true",
                    help="declare the clean half of a teacher-forcing workload tangent-free")
    ap.add_argument("--clock-seconds", type=float, default=2.0,
                    help="seconds of repeated steps after the timed ones, sampling the shader clock and board "
                         "power from sysfs (0: skip)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one device copy of this many MiB (counter calibration)")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_<workload>.json from two rocprofv3 counter_collection.csv "
                         "files (FETCH_SIZE run, WRITE_SIZE run) and exit; needs no GPU")
    args = ap.parse_args(argv)

    if args.record_traffic:
        from attention_jvp_causal_amd.workloads import BENCH_WORKLOAD

        wl = args.workload or BENCH_WORKLOAD
        cmd = ("rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv -- python3 bench.py "
               f"--workload {wl} --steps 3 --warmup 1 --cpu-heads 0 --clock-seconds 0 "
               f"--calib-copy-mib {args.calib_copy_mib or 1024}")
        print(json.dumps(record_traffic(wl, *args.record_traffic, args.calib_copy_mib or 1024, cmd)))
        return 0

    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; multi-GPU runs are not part of it",
                          "n_gpus": args.gpus}))
        return 2

    import torch

    import attention_jvp_causal_amd as aj
    from attention_jvp_causal_amd.workloads import BENCH_WORKLOAD, WORKLOADS, make_inputs

    w = WORKLOADS[args.workload or BENCH_WORKLOAD]
    inputs = make_inputs(w)
    dev = {n: t.to("cuda:0") for n, t in inputs.items()}
    desc = aj.attn_jvp_mask_desc_build(w.mask_kind, w.num_frames, w.frame_tokens, w.frames_per_chunk,
                                       head_dim=w.head_dim, dtype=w.dtype)
    if args.tangent_free:
        if not w.clean_tangent_zero:
            raise SystemExit(f"--tangent-free needs a workload whose clean half has zero tangents, not {w.name}")
        desc = aj.attn_jvp_mask_desc_tangent_free(desc, [(0, w.seq_len // 2)])
    if args.op == "kv":
        if w.mask_kind != "block_causal":
            raise SystemExit("--op kv needs a block-causal workload")
        chunk = w.frames_per_chunk * w.frame_tokens
        q_len = w.seq_len - ((w.seq_len - 1) // chunk) * chunk  # the last (possibly ragged) chunk
        desc = aj.attn_jvp_mask_desc_from_rects_kv(q_len, w.seq_len, [(0, q_len, 0, w.seq_len)],
                                                   head_dim=w.head_dim, dtype=w.dtype)
    pairs = desc.unmasked_pairs * w.batch * w.heads
    per_pair = {"jvp": 12.0, "fwd": 4.0, "bwd": 10.0, "kv": 4.0}[args.op]
    flop = per_pair * w.head_dim * pairs
    # FLOPs the kernels execute: fewer than the convention's on tangent-free
    # tiles; more for the gradients (14d)
    if args.op == "jvp":
        wk = desc.work()
        exec_flop = float(w.head_dim) * w.batch * w.heads * (12.0 * wk[0] + 8.0 * wk[1] + 4.0 * wk[2])
    elif args.op == "bwd":
        exec_flop = 14.0 * w.head_dim * pairs
    else:
        exec_flop = flop
    out_dtype = {None: None, "bf16": torch.bfloat16, "f32": torch.float32}[args.out_dtype]
    B, H, L, D = w.shape
    odt = out_dtype or dev["q"].dtype
    outs = (torch.empty((B, H, L, D), dtype=odt, device="cuda:0"),
            torch.empty((B, H, L, D), dtype=odt, device="cuda:0"),
            torch.empty((B, H, L), dtype=torch.float32, device="cuda:0"))
    args_ = [dev[n] for n in ("q", "k", "v", "tq", "tk", "tv")]
    v16 = uses_v16(w.dtype, w.head_dim, args.op) and not args.no_v16
    if v16:  # the fp16 copy buffers, allocated once outside the timed steps
        v16_bufs = tuple(torch.empty_like(dev[n], dtype=torch.float16) for n in ("v", "tv"))

    if args.op == "bwd":
        # forward outputs and a cotangent, made before the timed region
        o_f, lse_f = aj.attn_fwd(*args_[:3], desc, scale=w.scale)
        g = torch.Generator().manual_seed(1234)
        d_out = torch.randn(w.shape, generator=g, dtype=torch.float32).to(torch.bfloat16).to("cuda:0")
        grads = tuple(torch.empty((B, H, L, D), dtype=odt, device="cuda:0") for _ in range(3)) + (
            torch.empty((B, H, L), dtype=torch.float32, device="cuda:0"),)

    if args.op == "kv":
        q_chunk = dev["q"][:, :, w.seq_len - q_len:].contiguous()
        o_kv = torch.empty_like(q_chunk, dtype=odt)
        lse_kv = torch.empty((B, H, q_len), dtype=torch.float32, device="cuda:0")

    def step():
        if args.op == "kv":
            aj.attn_fwd_kv(q_chunk, dev["k"], dev["v"], desc, scale=w.scale, out_dtype=out_dtype, out=(o_kv, lse_kv))
        elif args.op == "jvp" and v16:
            aj.attn_jvp_fwd_v16(*args_, desc, scale=w.scale, out_dtype=out_dtype, out=outs, v16=v16_bufs)
        elif args.op == "jvp":
            aj.attn_jvp_fwd(*args_, desc, scale=w.scale, out_dtype=out_dtype, out=outs)
        elif args.op == "fwd":
            aj.attn_fwd(*args_[:3], desc, scale=w.scale, out_dtype=out_dtype, out=(outs[0], outs[2]))
        else:
            aj.attn_bwd(*args_[:3], o_f, d_out, lse_f, desc, scale=w.scale, out_dtype=out_dtype, out=grads)

    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()  # the binding launches on this stream
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in ev:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # Shader clock and board power under sustained load of the same step
    # (about 2 s after the timed steps, outside them: the clock settles over
    # a few hundred milliseconds, longer than the timed region).
    gpu_clock = None
    clock = ClockSampler()
    if clock.sclk and args.clock_seconds > 0:
        n_sus = max(1, int(args.clock_seconds * 1e3 / max(avg_ms_of(ev), 1e-3)))
        clock.start()
        for i in range(n_sus):
            step()
            if i % 8 == 7:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        gpu_clock = clock.stop()
        if gpu_clock:
            gpu_clock["steps"] = n_sus
    launch_ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    avg_ms = sum(launch_ms) / len(launch_ms)
    ms_per_step = wall * 1e3 / args.steps

    value = flop / (ms_per_step * 1e-3) / 1e12
    achieved = exec_flop / (avg_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_MFMA_TFLOPS
    kname = kernel_name(w.dtype, D, odt == torch.float32, args.op, args.tangent_free, w.scale, v16=v16)
    traffic = measured_traffic(w.name, kname.split(" + ")[-1])
    n_in, n_out = {"jvp": (6, 2), "fwd": (3, 1), "bwd": (5, 3), "kv": (2, 0)}[args.op]
    in_bytes = n_in * B * H * L * D * inputs["q"].element_size() + (B * H * L * 4 if args.op == "bwd" else 0)
    out_bytes = n_out * B * H * L * D * odt.itemsize + B * H * L * 4
    if args.op == "kv":  # K, V of the cache; q and o of the chunk; lse
        in_bytes += B * H * q_len * D * inputs["q"].element_size()
        out_bytes = B * H * q_len * (D * odt.itemsize + 4)
    if args.op != "jvp" or args.tangent_free:
        traffic = None  # counters are recorded for the plain JVP only

    cpu = None
    if args.cpu_heads > 0 and args.op == "jvp":
        cpu = cpu_baseline(w, inputs, min(args.cpu_heads, w.heads))

    metric = {"jvp": METRIC, "fwd": METRIC_FWD, "bwd": METRIC_BWD, "kv": METRIC_KV}[args.op]
    rec = {
        "metric": metric,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded i.i.d. Gaussian Q, K, V and tangents, Wan2.1 480p latent shapes)",
        "config": {
            "workload": w.name,
            "batch": B, "heads": H, "seq_len": L, "head_dim": D,
            "mask": f"{w.mask_kind} frames={w.num_frames} tokens_per_frame={w.frame_tokens} "
                    f"frames_per_chunk={w.frames_per_chunk}",
            "unmasked_pairs": pairs,
            "flop_per_step": flop,
            "op": args.op,
            "kv_cache": (f"last chunk of {q_len} queries over {L} cached keys" if args.op == "kv" else None),
            "v_tv_fp16_copies": ("attn_jvp_fwd_v16: a conversion kernel writes fp16 copies of V and tV, then the "
                                 "JVP kernel reads them; both inside the timed step" if v16 else None),
            "tangent_free": ("clean half [0, L/2) declared tangent-free; value counts 12d per pair, "
                             "roofline the executed 12d / 8d / 4d per pair by tile class")
                            if args.tangent_free else None,
            "executed_flop_per_step": exec_flop,
            "out_dtype": str(odt).replace("torch.", ""),
            "parallelism": "single GPU",
        },
        "pct_of_peak": round(100.0 * value / peak, 2),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": traffic,
            "kernel": kname,
            "launch_ms_avg": round(avg_ms, 4),
            "launch_ms_min": round(launch_ms[0], 4),
            "algorithmic_hbm_bytes": in_bytes + out_bytes,
        },
        "cpu_baseline": cpu,
        "gpu_clock": gpu_clock,
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
