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
    assert bench.kernel_name("bf16", 64, False, scale=0.125) == "attn_jvp_fwd_bf16_q32_kernel<64, false, true, true>"
    assert bench.kernel_name("bf16", 64, False, scale=0.1) == "attn_jvp_fwd_bf16_q32_kernel<64, false, true, false>"
    assert bench.kernel_name("bf16", 128, True, op="fwd") == "attn_jvp_fwd_bf16_q32_kernel<128, true, false, false>"
    assert bench.kernel_name("bf16", 128, False, op="bwd") == \
        "attn_bwd_dq32_kernel<128, false> + attn_bwd_dkdv_kernel<128, false>"
    assert bench.kernel_name("bf16", 128, False, tangent_free=True) == \
        "attn_jvp_fwd_bf16_q32_kernel<128, false, false, false> + attn_jvp_fwd_bf16_q16_kernel<128, false, true>"
    assert bench.kernel_name("f32", 64, True) == "attn_jvp_fwd_f32_kernel<64>"


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


def test_traffic_record_matches_the_kernel_sources():
    # bench.py reports roofline.traffic only while the counter record was
    # taken on the current kernel sources and flags; a kernel change needs a
    # new record (bench.py --record-traffic)
    from attention_jvp_causal_amd.workloads import BENCH_WORKLOAD

    path = os.path.join(ROOT, "profiles", f"traffic_{BENCH_WORKLOAD}.json")
    with open(path) as f:
        rec = json.load(f)
    assert rec["kernel_sha"] == bench.kernel_sha()
    assert rec["kernel"] == bench.kernel_name("bf16", 128, False)
    assert bench.measured_traffic(BENCH_WORKLOAD) == rec["bytes_per_launch"] > 0
