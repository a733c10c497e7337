"""Benchmark of the INT8-QK / FP8-PV attention forward on one MI355X.

One step = the whole hot path over one batch of synthetic input: the
preprocessing call (K sums / V maxima, K mean and V scales, INT8 and E4M3
codes) followed by the attention call.  The workload is the Wan-like video
self-attention shape B=1, H=40, Nq=Nkv=32760, D=128 (tail block of 120
tokens), Q/K/V ~ N(0,1) with one x8 outlier channel per head and a
per-channel key bias N(0, 2^2), drawn by testkit with seed 46.  Inputs are
resident in HBM before the timed region.

--workload picks another testkit workload: 6 is the short-query long-key
shape (split-KV with --num-splits 0), 7 the Wan-like workload under a seeded
block mask keeping half the 128x128 blocks (one step also rebuilds the block
table; FLOPs count the attended (query, key) pairs only).

Printed: one JSON line.  value = 4*B*H*Nq*Nkv*D / (time of one step), in
TFLOP/s; attention-only and quantize-only figures, the roofline of the
attention kernel (its average duration from HIP events recorded on the
stream it runs on) and the CPU oracle's rate on a bounded sample are
reported beside it.  gpu_clock holds the shader clock and board power
sampled from sysfs every 20 ms during the timed steps (null where the host
does not expose them for exactly one GPU, or where the steps take under
five sampling periods), and attention_only.frac_of_peak_at_sclk the
attention rate against the peak scaled to that clock.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s (4·B·H·Nq·Nkv·D), INT8-QK/FP8-PV, D=128; % of MFMA peak"
# (with --qk-format fp8 the same figure for the FP8 Q/K format)
PEAK_TFLOPS = 5000.0     # MI355X dense INT8 / FP8 MFMA
PEAK_HBM_GBS = 8000.0    # MI355X HBM3E
ATTN_KERNEL = "attn_pp_kernel"
SHORT_KERNEL = "attn_short_kernel"
# Sources that fix each attention kernel's code; a committed traffic record
# is used only while their digest matches the one it was measured with.
KERNEL_SOURCES = {
    ATTN_KERNEL: ("precision_flash_attention_amd/csrc/attn_fwd.hip",
                  "precision_flash_attention_amd/csrc/layout.h",
                  "precision_flash_attention_amd/csrc/kernels.h"),
    SHORT_KERNEL: ("precision_flash_attention_amd/csrc/attn_short.hip",
                   "precision_flash_attention_amd/csrc/layout.h",
                   "precision_flash_attention_amd/csrc/kernels.h"),
}
ATTN_SOURCES = KERNEL_SOURCES[ATTN_KERNEL]
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "attn_pp_kernel_wan_b1h40n32760_traffic.md")
COPY_BYTES = 1 << 30


def attn_algo_bytes(B, H, Nq, Nkv):
    """Codes + scales read and BF16 output written by one attention call."""
    nbq, nbk = -(-Nq // 128), -(-Nkv // 128)
    return B * H * (Nq * 128 + 2 * Nkv * 128 + 4 * (nbq + nbk + 128) + 2 * Nq * 128)


def quant_unique_bytes(B, H, Nq, Nkv):
    """BF16 Q/K/V read once and INT8/E4M3 codes written once."""
    return B * H * 128 * (Nq + 2 * Nkv) * 3


def attn_kernel_digest(kernel=ATTN_KERNEL):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_records():
    """Every traffic record committed under profiles/ (lines starting with
    'traffic-record: ' in the *_traffic.md summaries)."""
    import glob
    recs = []
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*_traffic.md"))):
        with open(path) as fh:
            recs += [json.loads(ln[len("traffic-record: "):]) for ln in fh if ln.startswith("traffic-record: ")]
    return recs


def measured_traffic(workload, qk_format, kernel=ATTN_KERNEL):
    """HBM bytes per launch of `kernel` from the committed FETCH_SIZE and
    WRITE_SIZE passes, each scaled by what the same counter read for a plain
    device copy of COPY_BYTES; None when there is no record for this kernel
    and workload or the kernel's sources changed since it was taken."""
    recs = traffic_records()
    digest = attn_kernel_digest(kernel)
    recs = [r for r in recs if r.get("kernel", ATTN_KERNEL) == kernel and r.get("kernel_digest") == digest
            and r.get("workload") == workload and r.get("qk_format", "int8") == qk_format]
    if not recs:
        return None
    rec = recs[0]
    fetch = rec["fetch_kib"] * rec["copy_bytes"] / rec["copy_fetch_kib"]
    write = rec["write_kib"] * rec["copy_bytes"] / rec["copy_write_kib"]
    return int(round(fetch + write))


def attention_kernel(B, H, Nq, Nkv, cus, sparse=False, q_smooth=False, splits=1, out_row_stride=None):
    """The kernel the library runs for a forward call of this shape: the
    short-KV kernel for 1-4 key tiles and more 256-query tiles than CUs
    (no block mask, no Q smoothing, one split, output rows 128 to 2^24
    elements apart), else attn_pp_kernel.  Mirrors the library's dispatch
    rule, for naming the kernel the roofline describes."""
    nbk = -(-Nkv // 128)
    os1 = H * 128 if out_row_stride is None else out_row_stride
    tiles = B * H * (-(-Nq // 256))
    if (not sparse and not q_smooth and splits == 1 and 1 <= nbk <= 4 and 128 <= os1 < (1 << 24)
            and cus < tiles < (1 << 30)):
        return SHORT_KERNEL
    return ATTN_KERNEL


PEAK_SCLK_MHZ = 2400.0    # the clock the 5.0 PFLOP/s peak is quoted at


def sclk_from_dpm(text):
    """Current shader clock in MHz from the text of a pp_dpm_sclk file: the
    level marked with '*'; None if no line is marked."""
    for ln in text.splitlines():
        if ln.rstrip().endswith("*"):
            num = "".join(ch for ch in ln.split(":", 1)[-1] if ch.isdigit() or ch == ".")
            return float(num) if num else None
    return None


def gpu_sysfs_dir():
    """The DRM device directory of the GPU when exactly one GPU on the host
    exposes its shader clock (pp_dpm_sclk); otherwise None (which card is
    cuda:0 is then not known)."""
    import glob
    cands = [d for d in sorted(glob.glob("/sys/class/drm/card*/device"))
             if os.path.exists(os.path.join(d, "pp_dpm_sclk"))]
    return cands[0] if len(cands) == 1 else None


class ClockSampler(threading.Thread):
    """Samples the shader clock and the board power from sysfs every
    `period` seconds while the timed steps run."""

    MIN_SAMPLES = 5

    def __init__(self, sysdir, period=0.02):
        super().__init__(daemon=True)
        self.sysdir, self.period = sysdir, period
        self.sclk, self.power = [], []
        self.stop = threading.Event()
        import glob
        pw = glob.glob(os.path.join(sysdir, "hwmon", "hwmon*", "power1_input"))
        self.power_file = pw[0] if len(pw) == 1 else None

    def run(self):
        while not self.stop.is_set():
            try:
                with open(os.path.join(self.sysdir, "pp_dpm_sclk")) as fh:
                    mhz = sclk_from_dpm(fh.read())
                if mhz is not None:
                    self.sclk.append(mhz)
                if self.power_file is not None:
                    with open(self.power_file) as fh:
                        self.power.append(int(fh.read().strip()) / 1e6)   # microwatts -> W
            except (OSError, ValueError):
                pass
            self.stop.wait(self.period)

    def summary(self):
        # a step sequence shorter than a few sampling periods is seen only
        # while the clock ramps up: no figure then
        if len(self.sclk) < self.MIN_SAMPLES:
            return None
        med = lambda xs: sorted(xs)[len(xs) // 2]  # noqa: E731
        return {"sclk_mhz_median": med(self.sclk), "sclk_mhz_min": min(self.sclk),
                "sclk_mhz_max": max(self.sclk), "power_w_median": med(self.power) if self.power else None,
                "samples": len(self.sclk), "source": "sysfs pp_dpm_sclk, hwmon power1_input"}


def copy_calibration(torch, dev):
    """Plain device-to-device copies of a known size, for scaling the HBM
    byte counters (FETCH_SIZE / WRITE_SIZE) of the other kernels."""
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


def cpu_baseline(cfg, q, k, v, rows_per_head, qk_format, block_mask=None, q_smooth=False):
    import numpy as np

    import oracle
    t0 = time.time()
    codes = oracle.quantize(q, k, v, qk_format=qk_format, q_smooth=q_smooth)
    t_quant = time.time() - t0
    stride = max(1, cfg.Nq // rows_per_head)
    rows = np.array([[b, h, i] for b in range(cfg.B) for h in range(cfg.H)
                     for i in range(0, cfg.Nq, stride)][: cfg.B * cfg.H * rows_per_head], np.int64)
    t0 = time.time()
    oracle.attention_rows(codes, cfg.softmax_scale, rows, block_mask=block_mask)
    t_rows = time.time() - t0
    total_rows = cfg.B * cfg.H * cfg.Nq
    t_step = t_quant + t_rows * total_rows / len(rows)
    return {
        "value": cfg.flops / t_step / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": (f"oracle quantize of the full workload ({t_quant:.2f} s) + oracle attention of "
                   f"{len(rows)} query rows ({rows_per_head} per head, {t_rows:.2f} s), scaled to all "
                   f"{total_rows} rows"),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=4, help="testkit workload index")
    ap.add_argument("--cpu-rows-per-head", type=int, default=320)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--qk-format", choices=("int8", "fp8"), default="int8",
                    help="Q/K code format: INT8 (scale amax/127) or E4M3 (scale amax/448)")
    ap.add_argument("--num-splits", type=int, default=0,
                    help="split-KV key ranges: 0 = the library's choice, 1 = none")
    ap.add_argument("--lse", action="store_true", help="also write the per-row LSE")
    ap.add_argument("--q-smooth", action="store_true",
                    help="Q smoothing per 128-token block with the Delta-S correction")
    ap.add_argument("--no-clock", action="store_true",
                    help="do not sample the shader clock and board power during the timed steps")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run 1 GiB device copies (reference kernel for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the path has no multi-GPU form in this library "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import precision_flash_attention_amd as sattn
    import testkit

    cfg = testkit.CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    q, k, v = testkit.make_inputs(cfg)
    to_dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    pbytes, wbytes = sattn.packed_bytes(cfg.B, cfg.H, cfg.Nq, cfg.Nkv, qk_format=args.qk_format,
                                        q_smooth=args.q_smooth)
    packed = torch.empty(pbytes, dtype=torch.uint8, device=dev)
    work = torch.empty(wbytes, dtype=torch.uint8, device=dev)
    out = torch.empty((cfg.B, cfg.Nq, cfg.H, 128), dtype=torch.bfloat16, device=dev)
    attend = sattn.fwd if cfg.Nq == cfg.Nkv else sattn.fwd_cross
    sparse = cfg.density is not None
    swb, splits = sattn.fwd_workspace_bytes(cfg.B, cfg.H, cfg.Nq, cfg.Nkv, 1 if sparse else args.num_splits)
    split_ws = torch.empty(swb, dtype=torch.uint8, device=dev) if swb else None
    mask_np = cfg.block_mask() if sparse else None
    mask_d = torch.from_numpy(mask_np).to(dev) if sparse else None
    lut_buf = torch.empty(sattn.block_lut_bytes(cfg.B, cfg.H, cfg.Nq, cfg.Nkv), dtype=torch.uint8,
                          device=dev) if sparse else None

    def step():
        p = sattn.quantize_qkv(qd, kd, vd, packed=packed, workspace=work, qk_format=args.qk_format,
                               q_smooth=args.q_smooth)
        ev[1].record()
        if sparse:
            # the block table is rebuilt every step, as for a mask predicted per step
            lut = sattn.block_lut(mask_d, cfg.Nq, cfg.Nkv, out=lut_buf)
            sattn.fwd_sparse(p, lut, cfg.softmax_scale, out=out, return_lse=args.lse)
        else:
            attend(p, cfg.softmax_scale, out=out, return_lse=args.lse, num_splits=args.num_splits,
                   workspace=split_ws)
        return p

    ev = [None, None, None]
    for _ in range(args.warmup):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        step()
    torch.cuda.synchronize()

    events = []
    sysdir = None if args.no_clock else gpu_sysfs_dir()
    sampler = ClockSampler(sysdir) if sysdir is not None else None
    if sampler is not None:
        sampler.start()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record()
        step()
        ev[2].record()
        events.append(ev)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    clock = None
    if sampler is not None:
        sampler.stop.set()
        sampler.join()
        clock = sampler.summary()
    ms_step = wall * 1e3 / args.steps
    t_quant = sum(e[0].elapsed_time(e[1]) for e in events) / args.steps
    t_attn = sum(e[1].elapsed_time(e[2]) for e in events) / args.steps
    t_attn_min = min(e[1].elapsed_time(e[2]) for e in events)
    t_attn_med = sorted(e[1].elapsed_time(e[2]) for e in events)[len(events) // 2]

    kernel = attention_kernel(cfg.B, cfg.H, cfg.Nq, cfg.Nkv, torch.cuda.get_device_properties(0).multi_processor_count,
                              sparse=sparse, q_smooth=args.q_smooth, splits=splits)
    flops = cfg.flops
    value = flops / (ms_step * 1e-3) / 1e12
    attn_tf = flops / (t_attn * 1e-3) / 1e12
    qbytes = quant_unique_bytes(cfg.B, cfg.H, cfg.Nq, cfg.Nkv)
    # the same rate against the peak scaled to the clock the GPU ran at
    frac_at_sclk = None
    if clock is not None:
        frac_at_sclk = round(attn_tf / (PEAK_TFLOPS * clock["sclk_mhz_median"] / PEAK_SCLK_MHZ), 4)
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8/fp8" if args.qk_format == "int8" else "fp8",
        "data": "synthetic",
        "config": dict(cfg.describe(), workload=cfg.name, softmax_scale=cfg.softmax_scale,
                       qk_format=args.qk_format, q_smooth=args.q_smooth, kv_splits=splits, lse=args.lse,
                       step="sattn_quantize_qkv + " + ("sattn_block_lut + sattn_fwd_sparse" if sparse else
                                                       "sattn_fwd" if cfg.Nq == cfg.Nkv else "sattn_fwd_cross")),
        "frac_of_peak": round(value / PEAK_TFLOPS, 4),
        "attended_fraction": round(flops / (4 * cfg.B * cfg.H * cfg.Nq * cfg.Nkv * 128), 4),
        "attention_only": {"ms": round(t_attn, 4), "ms_median": round(t_attn_med, 4), "ms_min": round(t_attn_min, 4),
                           "tflops": round(attn_tf, 2), "frac_of_peak": round(attn_tf / PEAK_TFLOPS, 4),
                           "frac_of_peak_at_sclk": frac_at_sclk},
        "quantize": {"ms": round(t_quant, 4), "unique_bytes": qbytes,
                     "gbs": round(qbytes / (t_quant * 1e-3) / 1e9, 1),
                     "frac_of_hbm_peak": round(qbytes / (t_quant * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
        "gpu_clock": clock,
        "roofline": {"bound": "mfma", "kernel": kernel, "achieved": round(attn_tf, 2),
                     "peak": PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(attn_tf / PEAK_TFLOPS, 4),
                     "traffic": measured_traffic(cfg.name, args.qk_format, kernel),
                     "algo_bytes": attn_algo_bytes(cfg.B, cfg.H, cfg.Nq, cfg.Nkv),
                     "kernel_digest": attn_kernel_digest(kernel)},
    }
    if args.copy_calibration:
        copy_calibration(torch, dev)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(cfg, q, k, v, args.cpu_rows_per_head, args.qk_format, mask_np,
                                           args.q_smooth)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
