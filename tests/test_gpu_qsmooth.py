"""GPU parity of Q smoothing with the Delta-S correction (the MHA v4 page's
Q-smoothing and Delta-S kernels) against ``oracle.quantize(q_smooth=True)``
and the oracle's attention on those codes: codes, scales and the Q block
means bit-exact; outputs and LSE within the bars of the format (the kernel
sums Delta-S in FP32 where the oracle is exact; that error is far below the
bar: ~2^-17 of sum_d |qmean_d kcode_d| ks per score)."""
import math

import numpy as np
import pytest

import oracle
import precision_flash_attention_amd as sattn
import testkit
from gpu_helpers import (MAX_ERR, MIN_COS, assert_codes_equal, from_dev, log, parity,
                         sample_rows, to_dev, workload)
from test_gpu_fp8qk import score_error_bound

pytestmark = pytest.mark.gpu
SCALE = 1.0 / math.sqrt(128.0)


def maxv(v):
    return float(np.abs(testkit.bf16_to_f32(v)).max())


def run(q, k, v, fmt="int8", num_splits=1, scale=SCALE):
    p = sattn.quantize_qkv(to_dev(q), to_dev(k), to_dev(v), qk_format=fmt, q_smooth=True)
    attend = sattn.fwd if p.Nq == p.Nkv else sattn.fwd_cross
    o, lse = attend(p, scale, return_lse=True, num_splits=num_splits)
    return from_dev(o), lse.cpu().numpy().astype(np.float64), p


def _decode(codes, fmt):
    return oracle.e4m3_decode(codes.view(np.uint8)) if fmt == "fp8" else codes.astype(np.float64)


def lse_bar_qs(c, scale):
    """Per-row LSE tolerance.  The kernel adds Delta-S, held in units u of
    the Q.K^T accumulator (u = qs, or 2^-20 for a block with qs = 0), to the
    FP32 view of the accumulator.  For INT8 that view carries the bias
    1.5 * 2^23, so the sum rounds to 1 unit (<= 0.5 u ks) inside the bias
    window, and the bias folded into the exponent offset moves the reference
    point by <= 0.75 u ks; past the window, and for FP8, the rounding is
    relative: 2^-24 of the sum, bounded here by 2^-20 of sum_d |q~_d||k~_d|
    (q~ = qcode qs + qmean, k~ = kcode ks)."""
    fmt = c.get("qk_format", "int8")
    qd = _decode(c["q8"], fmt)
    kd = _decode(c["k8"], fmt)
    Nq, Nkv = qd.shape[2], kd.shape[2]
    blk = np.arange(Nq) // 128
    qs = c["q_scale"].astype(np.float64)[:, :, blk]
    qm = c["q_mean"].astype(np.float64)[:, :, blk]                        # [B, H, Nq, D]
    km = c["k_mean"].astype(np.float64)[:, :, None, :]
    ks = c["k_scale"].astype(np.float64)[:, :, np.arange(Nkv) // 128]
    qt = np.abs(qd) * qs[..., None] + np.abs(qm)
    shift = (qt * np.abs(km)).sum(axis=3)
    smag = np.matmul(qt, np.ascontiguousarray(np.swapaxes(np.abs(kd) * ks[..., None], 2, 3))).max(axis=3)
    bar = 2.0 ** -20 * (shift + smag) * scale + 2e-4
    if fmt == "int8":
        u = np.where(qs > 0, qs, 2.0 ** -20)
        bar = bar + 1.25 * u * ks.max(axis=2)[:, :, None] * scale
    else:
        bar = bar + score_error_bound(c, scale)
    return bar


def check(q, k, v, what, fmt="int8", num_splits=1):
    o, lse, p = run(q, k, v, fmt, num_splits)
    c = oracle.quantize(q, k, v, qk_format=fmt, q_smooth=True)
    got = sattn.unpack_host(p)
    assert_codes_equal(got, c)
    assert np.array_equal(got["q_mean"].view(np.uint32), c["q_mean"].view(np.uint32))
    ref, ref_lse = oracle.attention(c, SCALE, return_lse=True)
    err, cs = parity(o, ref, maxv(v))
    bar = MAX_ERR if fmt == "int8" else MAX_ERR + 2.0 * score_error_bound(c, SCALE)
    lerr = np.abs(lse - ref_lse)
    lbar = lse_bar_qs(c, SCALE)
    log(f"  {what} [{fmt} + Q smoothing, splits {num_splits}]: out err {err:.3e} (bar {bar:.2e}) "
        f"cos {cs:.7f}; lse worst / bar {np.max(lerr / lbar):.3f}")
    assert err <= bar and cs >= MIN_COS, (err, bar, cs)
    assert np.all(lerr <= lbar)


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
@pytest.mark.parametrize("N", [1, 127, 129, 600])
def test_ragged_self(device, fmt, N):
    cfg = testkit.CONFIGS[4]
    q, k, v = testkit.make_inputs(cfg, seed=700 + N, H=3, Nq=N, Nkv=N)
    check(q, k, v, f"self N={N}", fmt)


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
@pytest.mark.parametrize("Nq,Nkv", [(300, 512), (1, 1000), (129, 1), (1000, 130)])
def test_cross_shapes(device, fmt, Nq, Nkv):
    cfg = testkit.CONFIGS[3]
    q, k, v = testkit.make_inputs(cfg, seed=15, B=2, H=3, Nq=Nq, Nkv=Nkv)
    check(q, k, v, f"cross {Nq}x{Nkv}", fmt)


def _offset_q(seed, Nq, H):
    rng = np.random.default_rng(seed)
    x = rng.normal(size=(1, Nq, H, 128)) + rng.normal(0, 4.0, size=(1, 1, H, 128))
    x = x.astype(np.float32)
    u = x.view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
def test_q_with_mean_offset(device, fmt):
    # the case smoothing is for: parity as everywhere, and the kernel output
    # closer to exact attention than without smoothing
    _, k, v = testkit.make_inputs(testkit.CONFIGS[1], seed=16, H=2, Nq=384, Nkv=512)
    q = _offset_q(17, 384, 2)
    check(q, k, v, "Q with a mean offset", fmt)
    o1, _, _ = run(q, k, v, fmt)
    p0 = sattn.quantize_qkv(to_dev(q), to_dev(k), to_dev(v), qk_format=fmt)
    o0 = from_dev(sattn.fwd_cross(p0, SCALE))
    exact = oracle.bruteforce(q, k, v, SCALE)
    e0 = np.abs(testkit.bf16_to_f32(o0) - exact).mean()
    e1 = np.abs(testkit.bf16_to_f32(o1) - exact).mean()
    log(f"    mean error to exact attention: smoothed {e1:.4e}, not smoothed {e0:.4e}")
    assert e1 < 0.9 * e0


@pytest.mark.parametrize("num_splits", [3, 0])
def test_split_kv(device, num_splits):
    cfg = testkit.CONFIGS[4]
    q, k, v = testkit.make_inputs(cfg, seed=18, H=2, Nq=200, Nkv=3000)
    o, lse, p = run(q, k, v, "int8", num_splits)
    c = oracle.quantize(q, k, v, q_smooth=True)
    ref, ref_lse = oracle.attention(c, SCALE, return_lse=True)
    err, cs = parity(o, ref, maxv(v))
    log(f"  split {num_splits} + Q smoothing: out err {err:.3e} cos {cs:.7f}")
    assert err <= MAX_ERR and cs >= 0.999
    assert np.all(np.abs(lse - ref_lse) <= lse_bar_qs(c, SCALE))


@pytest.mark.parametrize("cfg_index", [1, 2, 3, 4])
def test_full_size_codes_and_rows(device, cfg_index):
    log(f"Q smoothing at full size, workload {cfg_index}")
    cfg, q, k, v, _ = workload(cfg_index)
    p = sattn.quantize_qkv(to_dev(q), to_dev(k), to_dev(v), q_smooth=True)
    attend = sattn.fwd if p.Nq == p.Nkv else sattn.fwd_cross
    o = from_dev(attend(p, SCALE))
    c = oracle.quantize(q, k, v, q_smooth=True)
    got = sattn.unpack_host(p)
    assert_codes_equal(got, c)
    assert np.array_equal(got["q_mean"].view(np.uint32), c["q_mean"].view(np.uint32))
    rows = sample_rows(cfg.B, cfg.H, cfg.Nq, 8, seed=19 + cfg_index)
    ref, _, _ = oracle.attention_rows(c, SCALE, rows)
    err, cs = parity(o[rows[:, 0], rows[:, 2], rows[:, 1]], ref, maxv(v))
    log(f"  {cfg.name}, {len(rows)} rows: out err {err:.3e} cos {cs:.7f}")
    assert err <= MAX_ERR and cs >= MIN_COS


def test_sparse_with_smoothing_is_refused(device):
    import torch
    cfg = testkit.CONFIGS[1]
    q, k, v = testkit.make_inputs(cfg, Nq=256, Nkv=256)
    p = sattn.quantize_qkv(to_dev(q), to_dev(k), to_dev(v), q_smooth=True)
    lut = sattn.block_lut(torch.ones(1, 2, 2, 2, dtype=torch.uint8, device="cuda:0"), 256, 256)
    with pytest.raises(NotImplementedError):
        sattn.fwd_sparse(p, lut, SCALE)
