"""GPU parity of the LSE output and of split-KV (the FA4 autotuning page,
"Validation": output plus float32 LSE, split-KV behaviour).

LSE bar, per row, against the oracle's FP64 value: gpu_helpers.lse_bar,
derived from the kernel's FP32 steps (dequantisation constant, row maximum,
the K-mean shift's dot product, the FP32 row sum and its rescales), plus the
row's FP8 score-error bound in the FP8 Q/K format.

Outputs under split-KV: each key range quantizes 448 p against its own
running maximum, so its P codes sit on another grid than the oracle's (which
quantizes against the row's final maximum, as the unsplit kernel does after
its first tiles).  The two roundings are then nearly independent, and on
rows that average many keys (small outputs) the cosine to the oracle can fall
below 0.9995 while the split result is closer to exact attention than the
oracle is (measured: 64 x 4608 cross-attention, cosine to exact 0.99927 with
8 ranges, 0.99924 unsplit, 0.99922 for the oracle).  So a split run (more than
one range) must meet the max-error bar against the oracle, and, where exact
FP64 attention is computed, be at least as close to it as the oracle (cosine
within 2e-4); by the triangle inequality for angles its cosine to the oracle
is then at least 2 c^2 - 1 (c: the oracle's cosine to exact), asserted too."""
import math

import numpy as np
import pytest

import oracle
import precision_flash_attention_amd as sattn
import testkit
from gpu_helpers import (MAX_ERR, MIN_COS, from_dev, log, lse_bar, out_bar, parity, row_errors,
                         sample_rows_strided, to_dev)

pytestmark = pytest.mark.gpu
SCALE = 1.0 / math.sqrt(128.0)


def maxv(v):
    return float(np.abs(testkit.bf16_to_f32(v)).max())


def run(q, k, v, fmt="int8", num_splits=0, scale=SCALE):
    p = sattn.quantize_qkv(to_dev(q), to_dev(k), to_dev(v), qk_format=fmt)
    attend = sattn.fwd if p.Nq == p.Nkv else sattn.fwd_cross
    o, lse = attend(p, scale, return_lse=True, num_splits=num_splits)
    return from_dev(o), lse.cpu().numpy().astype(np.float64)


def cos(a, b):
    a = a.ravel().astype(np.float64)
    b = b.ravel().astype(np.float64)
    return float(a @ b / np.sqrt((a @ a) * (b @ b)))


def check(q, k, v, what, fmt="int8", num_splits=0, scale=SCALE):
    o, lse = run(q, k, v, fmt, num_splits, scale)
    used = sattn.fwd_workspace_bytes(q.shape[0], q.shape[2], q.shape[1], k.shape[1], num_splits)[1]
    c = oracle.quantize(q, k, v, qk_format=fmt)
    ref, ref_lse = oracle.attention(c, scale, return_lse=True)
    err, cs = parity(o, ref, maxv(v))
    ratio = float(np.max(row_errors(o, ref, maxv(v)) / out_bar(c, scale)))
    lerr = np.abs(lse - ref_lse)
    lbar = lse_bar(c, scale)
    log(f"  {what} [{fmt}, splits {num_splits} -> {used}]: out err {err:.3e} (worst / bar {ratio:.3f}) "
        f"cos to the oracle {cs:.7f}; lse err max {lerr.max():.2e}, worst / bar {np.max(lerr / lbar):.3f}")
    assert ratio <= 1.0, ratio
    assert np.all(lerr <= lbar)
    if used == 1:
        assert cs >= MIN_COS, cs
    else:
        exact = oracle.bruteforce(q, k, v, scale)
        c_k = cos(testkit.bf16_to_f32(o), exact)
        c_o = cos(testkit.bf16_to_f32(ref), exact)
        log(f"    split run, cosine: to the oracle {cs:.7f}; to exact attention: kernel {c_k:.6f}, "
            f"oracle {c_o:.6f}")
        assert c_k >= c_o - 2e-4
        assert cs >= 2.0 * (c_o - 2e-4) ** 2 - 1.0
    return o, lse


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
@pytest.mark.parametrize("N", [1, 127, 129, 600])
def test_lse_self_ragged(device, fmt, N):
    cfg = testkit.CONFIGS[4]
    q, k, v = testkit.make_inputs(cfg, seed=500 + N, H=3, Nq=N, Nkv=N)
    check(q, k, v, f"self N={N}", fmt, num_splits=1)


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
@pytest.mark.parametrize("Nq,Nkv", [(300, 512), (1, 1000), (129, 1)])
def test_lse_cross(device, fmt, Nq, Nkv):
    cfg = testkit.CONFIGS[3]
    q, k, v = testkit.make_inputs(cfg, seed=14, B=2, H=3, Nq=Nq, Nkv=Nkv)
    check(q, k, v, f"cross {Nq}x{Nkv}", fmt, num_splits=1)


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
@pytest.mark.parametrize("num_splits", [0, 2, 4, 7, 40])
def test_split_kv_short_queries_long_keys(device, fmt, num_splits):
    # 40 key tiles (the last holding 8 keys): 7 -> 7 ranges of 6 tiles (the
    # last range 4), 40 -> one tile each (the tail tile alone), 0 -> auto
    cfg = testkit.CONFIGS[4]
    q, k, v = testkit.make_inputs(cfg, seed=77, H=4, Nq=200, Nkv=5000)
    used = sattn.fwd_workspace_bytes(1, 4, 200, 5000, num_splits)[1]
    log(f"split-KV Nq=200 Nkv=5000 H=4: num_splits {num_splits} -> {used} ranges")
    assert used == {0: 5, 2: 2, 4: 4, 7: 7, 40: 40}[num_splits]
    check(q, k, v, "self 200x5000 (cross call)", fmt, num_splits)


@pytest.mark.parametrize("num_splits", [3, 0])
def test_split_kv_self_call(device, num_splits):
    cfg = testkit.CONFIGS[2]
    q, k, v = testkit.make_inputs(cfg, seed=78, H=2, Nq=1100, Nkv=1100)
    check(q, k, v, "self 1100", "int8", num_splits)


@pytest.mark.parametrize("cfg_index,shape", [(3, dict(seed=11, B=2, H=3, Nq=64, Nkv=4608)),
                                              (2, dict(seed=5, H=2, Nq=64, Nkv=8192)),
                                              (3, dict(seed=12, B=2, H=3, Nq=1, Nkv=1000))])
@pytest.mark.parametrize("num_splits", [2, 8])
def test_split_averaging_rows_closer_to_exact(device, cfg_index, shape, num_splits):
    # rows that average thousands of keys: the case where the split's P grid
    # moves the output away from the oracle but not away from exact attention
    q, k, v = testkit.make_inputs(testkit.CONFIGS[cfg_index], **shape)
    check(q, k, v, f"averaging {shape['Nq']}x{shape['Nkv']}", "int8", num_splits)


def test_split_matches_unsplit_closely(device):
    # a different running maximum per key range changes which 448 p values
    # round up or down, nothing else
    cfg = testkit.CONFIGS[4]
    q, k, v = testkit.make_inputs(cfg, seed=79, H=2, Nq=64, Nkv=4000)
    o1, l1 = run(q, k, v, num_splits=1)
    o5, l5 = run(q, k, v, num_splits=5)
    err, cs = parity(o5, o1, maxv(v))
    log(f"  split 5 vs 1: out err {err:.3e} cos {cs:.7f}; lse diff {np.abs(l5 - l1).max():.2e}")
    assert err <= MAX_ERR and cs >= 0.9995
    c = oracle.quantize(q, k, v)
    assert np.all(np.abs(l5 - l1) <= 2 * lse_bar(c, SCALE))


def test_split_with_strided_output_and_3d(device):
    import torch
    cfg = testkit.CONFIGS[3]
    q, k, v = testkit.make_inputs(cfg, seed=80, B=1, H=4, Nq=100, Nkv=3000)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    p = sattn.quantize_qkv(qd, kd, vd)
    ref, ref_lse = sattn.fwd_cross(p, SCALE, return_lse=True, num_splits=6)
    wide = torch.full((1, 100, 7, 128), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    out = wide[:, :, 1:5]
    _, lse = sattn.fwd_cross(p, SCALE, out=out, return_lse=True, num_splits=6)
    assert torch.equal(out, ref) and torch.equal(lse, ref_lse)
    assert torch.isnan(wide[:, :, :1]).all() and torch.isnan(wide[:, :, 5:]).all()
    o3, l3 = sattn.attention(qd[0], kd[0], vd[0], SCALE, return_lse=True, num_splits=6)
    assert o3.shape == (100, 4, 128) and l3.shape == (4, 100)
    assert torch.equal(o3, ref[0]) and torch.equal(l3, ref_lse[0])
    # a caller-provided workspace gives the same result; a short one is refused
    wb, used = sattn.fwd_workspace_bytes(1, 4, 100, 3000, 6)
    ws = torch.empty(wb, dtype=torch.uint8, device="cuda:0")
    o_ws = sattn.fwd_cross(p, SCALE, num_splits=6, workspace=ws)
    assert used == 6 and torch.equal(o_ws, ref)
    with pytest.raises(ValueError):
        sattn.fwd_cross(p, SCALE, num_splits=6, workspace=ws[: wb - 256])


def test_split_deterministic(device):
    import torch
    cfg = testkit.CONFIGS[4]
    q, k, v = testkit.make_inputs(cfg, seed=81, H=3, Nq=256, Nkv=6000)
    p = sattn.quantize_qkv(to_dev(q), to_dev(k), to_dev(v))
    a, la = sattn.fwd_cross(p, SCALE, return_lse=True, num_splits=0)
    b, lb = sattn.fwd_cross(p, SCALE, return_lse=True, num_splits=0)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
def test_short_query_wan_shape_sampled(device, fmt):
    # the Wan-like recipe with 256 queries against its 32760 keys: 40
    # workgroups without a split, 240 with the automatic 6 ranges
    cfg = testkit.CONFIGS[4]
    q, k, v = testkit.make_inputs(cfg, seed=82, Nq=256)
    assert sattn.fwd_workspace_bytes(1, 40, 256, 32760, 0)[1] == 6
    o, lse = run(q, k, v, fmt, num_splits=0)
    c = oracle.quantize(q, k, v, qk_format=fmt)
    rows = sample_rows_strided(1, 40, 256, 1, seed=3)  # every row
    ref, _, _, ref_lse = oracle.attention_rows(c, SCALE, rows, return_lse=True)
    got = o[rows[:, 0], rows[:, 2], rows[:, 1]]
    err, cs = parity(got, ref, maxv(v))
    ratio = float(np.max(row_errors(got, ref, maxv(v)) / out_bar(c, SCALE, rows)))
    lerr = np.abs(lse[rows[:, 0], rows[:, 1], rows[:, 2]] - ref_lse)
    lbar = lse_bar(c, SCALE, rows)
    # exact FP64 attention of the sampled rows from the BF16 inputs
    qf, kf, vf = (testkit.bf16_to_f32(t).astype(np.float64) for t in (q, k, v))
    exact = np.empty((len(rows), 128))
    for n, (b, h, i) in enumerate(rows):
        s = SCALE * (kf[b, :, h] @ qf[b, i, h])
        w = np.exp(s - s.max())
        exact[n] = (w @ vf[b, :, h]) / w.sum()
    c_k = cos(testkit.bf16_to_f32(got), exact)
    c_o = cos(testkit.bf16_to_f32(ref), exact)
    log(f"  wan 256x32760 [{fmt}], {len(rows)} rows: out err {err:.3e} (worst / bar {ratio:.3f}) "
        f"cos to the oracle {cs:.7f}; lse worst / bar {np.max(lerr / lbar):.3f}; "
        f"vs exact: kernel {c_k:.6f}, oracle {c_o:.6f}")
    assert ratio <= 1.0 and cs >= 2.0 * (c_o - 2e-4) ** 2 - 1.0
    assert c_k >= c_o - 2e-4
    assert np.all(lerr <= lbar)
