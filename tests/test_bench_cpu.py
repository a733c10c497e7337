"""Host logic of bench.py (CPU): algorithmic byte counts, the HBM traffic
record and its digest gate, and the refusal of more than one GPU."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
WAN = "wan-like video self-attention"


def test_algorithmic_bytes_of_the_wan_workload():
    B, H, N = 1, 40, 32760
    nb = -(-N // 128)
    # Q, K and V codes (1 byte each), the Q/K block scales and the V channel
    # scales (4 bytes each), and the BF16 output
    want = B * H * (3 * N * 128 + 4 * (2 * nb + 128) + 2 * N * 128)
    assert bench.attn_algo_bytes(B, H, N, N) == want == 838758400
    # BF16 Q, K, V read once; one code byte each written
    assert bench.quant_unique_bytes(B, H, N, N) == 3 * B * H * N * 128 * 3 == 1509580800


def _records():
    with open(bench.TRAFFIC_RECORD) as fh:
        return [json.loads(ln[len("traffic-record: "):]) for ln in fh if ln.startswith("traffic-record: ")]


def test_every_profile_record_is_read():
    recs = bench.traffic_records()
    assert all(r in recs for r in _records())
    assert all(r.get("kernel", bench.ATTN_KERNEL) in bench.KERNEL_SOURCES for r in recs)


def test_kernel_named_by_the_dispatch_rule():
    k = bench.attention_kernel
    # text cross-attention: 4 key tiles, 10240 query tiles on 256 CUs
    assert k(2, 40, 32760, 512, 256) == bench.SHORT_KERNEL
    assert k(2, 40, 32760, 513, 256) == bench.ATTN_KERNEL      # 5 key tiles
    assert k(1, 40, 32760, 32760, 256) == bench.ATTN_KERNEL    # Wan-like
    assert k(1, 2, 256, 256, 256) == bench.ATTN_KERNEL         # 2 query tiles
    assert k(1, 1, 256 * 256, 1, 256) == bench.ATTN_KERNEL     # exactly one tile per CU
    assert k(1, 1, 256 * 257, 1, 256) == bench.SHORT_KERNEL
    assert k(2, 40, 32760, 512, 256, sparse=True) == bench.ATTN_KERNEL
    assert k(2, 40, 32760, 512, 256, q_smooth=True) == bench.ATTN_KERNEL
    assert k(2, 40, 32760, 512, 256, splits=2) == bench.ATTN_KERNEL
    assert k(2, 40, 32760, 512, 256, out_row_stride=64) == bench.ATTN_KERNEL


def test_traffic_record_is_reported_only_for_its_kernel():
    recs = [r for r in _records() if r["workload"] == WAN]
    assert {r["qk_format"] for r in recs} == {"int8", "fp8"}
    digest = bench.attn_kernel_digest()
    for r in recs:
        got = bench.measured_traffic(WAN, r["qk_format"])
        if r["kernel_digest"] != digest:
            # counters of an older kernel are not reported
            assert got is None
            continue
        # each counter scaled by what it read for a device copy of known size
        want = (r["fetch_kib"] * r["copy_bytes"] / r["copy_fetch_kib"]
                + r["write_kib"] * r["copy_bytes"] / r["copy_write_kib"])
        assert got == int(round(want))
        # at least the algorithmic bytes, the BF16 output written exactly once
        assert got >= bench.attn_algo_bytes(1, 40, 32760, 32760)
        assert abs(r["write_kib"] * 1024 - 2 * 32760 * 40 * 128) < 1024


def test_traffic_is_null_for_other_kernels_and_workloads(monkeypatch):
    assert bench.measured_traffic("text cross-attention", "int8") is None
    assert bench.measured_traffic(WAN, "int8", bench.SHORT_KERNEL) is None
    monkeypatch.setattr(bench, "attn_kernel_digest", lambda kernel=bench.ATTN_KERNEL: "0" * 16)
    assert bench.measured_traffic(WAN, "int8") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_shader_clock_parser():
    # the current clock between levels ("S:" line) and on a level
    assert bench.sclk_from_dpm("S: 120Mhz *\n0: 500Mhz\n1: 2400Mhz\n") == 120.0
    assert bench.sclk_from_dpm("0: 500Mhz\n1: 2400Mhz *\n") == 2400.0
    assert bench.sclk_from_dpm("0: 500Mhz\n1: 2400Mhz\n") is None
    assert bench.sclk_from_dpm("") is None


def test_clock_summary_needs_several_samples(tmp_path):
    s = bench.ClockSampler(str(tmp_path))
    s.sclk = [783.0]
    assert s.summary() is None
    s.sclk = [1700.0, 1800.0, 1750.0, 1900.0, 1200.0]
    s.power = [1000.0] * 5
    got = s.summary()
    assert got["sclk_mhz_median"] == 1750.0 and got["sclk_mhz_min"] == 1200.0 and got["samples"] == 5
