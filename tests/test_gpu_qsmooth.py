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
from gpu_helpers import (FULL_SIZE_STRIDE, MIN_COS, assert_codes_equal, check_rows, from_dev, log,
                         lse_bar, out_bar, parity, row_errors, sample_rows_strided, to_dev, workload)

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


def cos(a, b):
    a = a.ravel().astype(np.float64)
    b = b.ravel().astype(np.float64)
    return float(a @ b / np.sqrt((a @ a) * (b @ b)))


def check(q, k, v, what, fmt="int8", num_splits=1):
    """Codes, scales and means bit-exact; every row within its output bar
    and its LSE bar (gpu_helpers.lse_bar, which counts the FP32 sum of the
    accumulator and Delta-S); the cosine to the oracle >= 0.9995 without a
    split.  A split run quantizes P against each key range's own maximum,
    so it is held instead to staying as close to exact FP64 attention as the
    oracle (its cosine to the oracle is then at least 2 c^2 - 1, c the
    oracle's cosine to exact attention)."""
    o, lse, p = run(q, k, v, fmt, num_splits)
    c = oracle.quantize(q, k, v, qk_format=fmt, q_smooth=True)
    got = sattn.unpack_host(p)
    assert_codes_equal(got, c)
    assert np.array_equal(got["q_mean"].view(np.uint32), c["q_mean"].view(np.uint32))
    ref, ref_lse = oracle.attention(c, SCALE, return_lse=True)
    err, cs = parity(o, ref, maxv(v))
    ratio = float(np.max(row_errors(o, ref, maxv(v)) / out_bar(c, SCALE)))
    lerr = np.abs(lse - ref_lse)
    lbar = lse_bar(c, SCALE)
    used = sattn.fwd_workspace_bytes(q.shape[0], q.shape[2], q.shape[1], k.shape[1], num_splits)[1]
    log(f"  {what} [{fmt} + Q smoothing, splits {num_splits} -> {used}]: out err {err:.3e} "
        f"(worst / bar {ratio:.3f}) cos to the oracle {cs:.7f}; lse worst / bar {np.max(lerr / lbar):.3f}")
    assert ratio <= 1.0, ratio
    assert np.all(lerr <= lbar)
    if used == 1:
        assert cs >= MIN_COS, cs
    else:
        exact = oracle.bruteforce(q, k, v, SCALE)
        c_k = cos(testkit.bf16_to_f32(o), exact)
        c_o = cos(testkit.bf16_to_f32(ref), exact)
        log(f"    split run, cosine to exact attention: kernel {c_k:.6f}, oracle {c_o:.6f}")
        assert c_k >= c_o - 2e-4
        assert cs >= 2.0 * (c_o - 2e-4) ** 2 - 1.0


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


def _bf16(x):
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
def test_degenerate_blocks(device, fmt):
    # Q block 1: 128 equal tokens (qs = 0, all-zero codes: the scores are
    # the block mean's alone); block 2: one channel at 3000 over a residual
    # of about 1e-3 (a mean of ~1e8 code units, past the INT8 accumulator
    # unless counted in a coarser unit); block 0 ordinary
    rng = np.random.default_rng(31)
    H, Nq, Nkv = 2, 300, 400
    q = rng.normal(size=(1, Nq, H, 128)).astype(np.float32)
    q[:, 128:256] = rng.normal(size=(1, 1, H, 128))
    q[:, 256:] = rng.normal(0.0, 1e-3, size=(1, Nq - 256, H, 128))
    q[:, 256:, :, 0] = 3000.0
    _, k, v = testkit.make_inputs(testkit.CONFIGS[4], seed=32, H=H, Nq=Nq, Nkv=Nkv)
    check(_bf16(q), k, v, "degenerate Q blocks", fmt)


@pytest.mark.parametrize("num_splits", [3, 0])
def test_split_kv(device, num_splits):
    cfg = testkit.CONFIGS[4]
    q, k, v = testkit.make_inputs(cfg, seed=18, H=2, Nq=200, Nkv=3000)
    check(q, k, v, "split 200x3000", "int8", num_splits)


@pytest.mark.parametrize("cfg_index", [1, 2, 3, 4, 5])
def test_full_size_codes_and_rows(device, cfg_index):
    log(f"Q smoothing at full size, workload {cfg_index}")
    cfg, q, k, v, _ = workload(cfg_index)
    p = sattn.quantize_qkv(to_dev(q), to_dev(k), to_dev(v), q_smooth=True)
    attend = sattn.fwd if p.Nq == p.Nkv else sattn.fwd_cross
    o = from_dev(attend(p, SCALE))
    c = oracle.quantize(q, k, v, q_smooth=True)
    got = sattn.unpack_host(p)
    del p
    assert_codes_equal(got, c)
    assert np.array_equal(got["q_mean"].view(np.uint32), c["q_mean"].view(np.uint32))
    stride = FULL_SIZE_STRIDE.get(cfg_index, 1) * 4
    rows = sample_rows_strided(cfg.B, cfg.H, cfg.Nq, stride, seed=19 + cfg_index)
    ref, _, _ = oracle.attention_rows(c, SCALE, rows)
    check_rows(o[rows[:, 0], rows[:, 2], rows[:, 1]], ref, v, out_bar(c, SCALE, rows),
               f"{cfg.name}, {len(rows)} rows")


def test_sparse_with_smoothing_is_refused(device):
    import torch
    cfg = testkit.CONFIGS[1]
    q, k, v = testkit.make_inputs(cfg, Nq=256, Nkv=256)
    p = sattn.quantize_qkv(to_dev(q), to_dev(k), to_dev(v), q_smooth=True)
    lut = sattn.block_lut(torch.ones(1, 2, 2, 2, dtype=torch.uint8, device="cuda:0"), 256, 256)
    with pytest.raises(NotImplementedError):
        sattn.fwd_sparse(p, lut, SCALE)
