"""Host-side checks of bench.py that need no GPU: the one-GPU contract, the
kernel names the roofline reports, and the sysfs clock sampler's parsing."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    rec = json.loads(r.stdout.strip().splitlines()[-1])
    assert rec["n_gpus"] == 2 and "one GPU" in rec["error"]


def test_kernel_names_follow_the_dispatch():
    assert bench.kernel_name("bf16", 128, False) == "attn_jvp_fwd_bf16_q16_kernel<128, false, false>"
    assert bench.kernel_name("bf16", 64, False, scale=0.125) == \
        "attn_jvp_fwd_bf16_q32_kernel<64, false, true, true, false, 4, false>"
    assert bench.kernel_name("bf16", 64, False, scale=0.1) == \
        "attn_jvp_fwd_bf16_q32_kernel<64, false, true, false, false, 4, false>"
    # attn_jvp_fwd_v16: the conversion kernel, then the instance reading the fp16 copies
    assert bench.kernel_name("bf16", 64, False, scale=0.125, v16=True) == \
        "bf16_to_f16_kv_kernel<64> + attn_jvp_fwd_bf16_q32_kernel<64, false, true, true, false, 4, true>"
    assert bench.uses_v16("bf16", 64) and not bench.uses_v16("bf16", 128) and not bench.uses_v16("bf16", 64, "fwd")
    # the primal forward (and the KV step) at d = 128 runs 8-wave, 256-row tasks
    assert bench.kernel_name("bf16", 128, True, op="fwd") == \
        "attn_jvp_fwd_bf16_q32_kernel<128, true, false, false, false, 8, false>"
    assert bench.kernel_name("bf16", 128, False, op="kv") == \
        "attn_jvp_fwd_bf16_q32_kernel<128, false, false, false, false, 8, false>"
    assert bench.kernel_name("bf16", 64, False, op="fwd") == \
        "attn_jvp_fwd_bf16_q32_kernel<64, false, false, false, false, 4, false>"
    assert bench.kernel_name("bf16", 128, False, op="bwd") == \
        "attn_bwd_dq32_kernel<128, false> + attn_bwd_dkdv_kernel<128, false>"
    assert bench.kernel_name("bf16", 64, False, op="bwd") == \
        "attn_bwd_dq32_kernel<64, false> + attn_bwd_dkdv32_kernel<64, false>"
    # the primal-only query tiles of a tangent-free JVP keep 4-wave tasks
    assert bench.kernel_name("bf16", 128, False, tangent_free=True) == \
        "attn_jvp_fwd_bf16_q32_kernel<128, false, false, false, false, 4, false> + " \
        "attn_jvp_fwd_bf16_q16_kernel<128, false, true>"
    assert bench.kernel_name("bf16", 64, False, tangent_free=True) == \
        "attn_jvp_fwd_bf16_q32_kernel<64, false, false, false, false, 4, false> + " \
        "attn_jvp_fwd_bf16_q32_kernel<64, false, true, true, true, 4, false>"
    assert bench.kernel_name("bf16", 64, False, tangent_free=True, v16=True) == \
        "attn_jvp_fwd_bf16_q32_kernel<64, false, false, false, false, 4, false> + bf16_to_f16_kv_kernel<64> + " \
        "attn_jvp_fwd_bf16_q32_kernel<64, false, true, true, true, 4, true>"
    assert bench.kernel_name("f32", 64, True) == "attn_jvp_fwd_f32_kernel<64>"


def test_every_launched_kernel_has_a_code_hash():
    # the build records a hash of each kernel's generated code; every forward
    # instance bench.py can name must be among them
    for D, scale in ((128, None), (64, 0.125), (64, 0.1)):
        for tf in (False, True):
            for v16 in ((False, True) if D == 64 else (False,)):
                for name in bench.kernel_name("bf16", D, False, tangent_free=tf, scale=scale, v16=v16).split(" + "):
                    assert bench.kernel_isa_sha(name), name
        for op in ("fwd", "kv"):
            assert bench.kernel_isa_sha(bench.kernel_name("bf16", D, False, op=op)), (D, op)
        for name in bench.kernel_name("bf16", D, False, op="bwd").split(" + "):
            assert bench.kernel_isa_sha(name), name


def test_clock_sampler_reads_the_starred_level(tmp_path):
    sclk = tmp_path / "pp_dpm_sclk"
    sclk.write_text("0: 500Mhz\n1: 2186Mhz *\n2: 2400Mhz\n")
    power = tmp_path / "power1_input"
    power.write_text("1308000000\n")
    c = bench.ClockSampler(period_s=0.001)
    c.sclk, c.power = str(sclk), str(power)
    assert c._read() == (2186, 1308.0)
    c.start()
    import time

    time.sleep(0.02)
    rec = c.stop()
    assert rec["sclk_mhz_median"] == 2186 and rec["board_power_w_median"] == 1308.0 and rec["samples"] >= 1


def test_clock_sampler_without_sysfs_reports_nothing():
    c = bench.ClockSampler()
    c.sclk = c.power = None
    c.start()
    assert c.stop() is None


def test_traffic_records_match_the_kernel_code():
    # bench.py reports roofline.traffic only while the counter record was
    # taken on the kernel code the build produced (the hash of its gfx950
    # instructions); a change to that code needs a new record
    # (bench.py --record-traffic).  The bench workload must have one.
    import glob

    from attention_jvp_causal_amd.workloads import BENCH_WORKLOAD, WORKLOADS

    paths = sorted(glob.glob(os.path.join(ROOT, "profiles", "traffic_*.json")))
    assert os.path.join(ROOT, "profiles", f"traffic_{BENCH_WORKLOAD}.json") in paths
    for path in paths:
        with open(path) as f:
            rec = json.load(f)
        w = WORKLOADS[rec["workload"]]
        kname = bench.kernel_name(w.dtype, w.head_dim, False, scale=w.scale,
                                  v16=bench.uses_v16(w.dtype, w.head_dim)).split(" + ")[-1]
        assert rec["kernel"] == kname, path
        assert rec["kernel_isa"] == bench.kernel_isa_sha(rec["kernel"]), path
        assert bench.measured_traffic(w.name, kname) == rec["bytes_per_launch"] > 0, path
        assert bench.measured_traffic(w.name, "another_kernel<1>") is None


def test_counter_profiles_name_the_kernel_code_that_builds():
    # every profiles/*.md names the code hash of the kernel it measured; it
    # must be the hash of a kernel this build produces (re-profile after a
    # change to a kernel's code), and its title must name that kernel
    import glob
    import re

    with open(os.path.join(ROOT, "attention_jvp_causal_amd", "libattnjvp.isa.json")) as f:
        isa = json.load(f)
    paths = sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md")))
    assert paths
    for path in paths:
        with open(path) as f:
            text = f.read()
        m = re.search(r"Kernel code hash.*?\): `([0-9a-f]{16})`", text)
        assert m, path
        title = re.match(r"# `([^`]+)`", text).group(1)
        names = [k for k, v in isa.items() if v == m.group(1)]
        assert any(f"aj::{title}(" in k for k in names), (path, title, m.group(1))
