"""GPU attention parity against the oracle: every workload at its full size
(full output for the small ones, sampled rows for the large ones), ragged
tails, cross shapes, strided outputs, closed-form cases and determinism.

Bar: max |O_gpu - O_oracle| <= 2e-2 * max|V| and cosine >= 0.9995 (FP64,
over the compared elements)."""
import math

import numpy as np
import pytest

import oracle
import precision_flash_attention_amd as sattn
import testkit
from gpu_helpers import (FULL_SIZE_STRIDE, MAX_ERR, MIN_COS, from_dev, log, parity, sample_rows_strided, to_dev,
                         workload)

pytestmark = pytest.mark.gpu
SCALE = 1.0 / math.sqrt(128.0)


def gpu_attention(q, k, v, scale=SCALE):
    p = sattn.quantize_qkv(to_dev(q), to_dev(k), to_dev(v))
    o = sattn.fwd(p, scale) if p.Nq == p.Nkv else sattn.fwd_cross(p, scale)
    return from_dev(o)


def maxv(v):
    return float(np.abs(testkit.bf16_to_f32(v)).max())


def check(o_gpu, o_orc, v, what):
    err, c = parity(o_gpu, o_orc, maxv(v))
    log(f"  {what}: max err / max|V| = {err:.3e}, cos = {c:.7f}")
    assert err <= MAX_ERR and c >= MIN_COS, (err, c)


@pytest.mark.parametrize("cfg_index", [1, 2])
def test_full_output(device, cfg_index):
    log(f"attention parity (full), workload {cfg_index}")
    cfg, q, k, v, codes = workload(cfg_index)
    o = gpu_attention(q, k, v)
    check(o, oracle.attention(codes, SCALE), v, cfg.name)


@pytest.mark.parametrize("cfg_index", [3, 4, 5])
def test_sampled_rows_full_size(device, cfg_index):
    log(f"attention parity (sampled rows), workload {cfg_index}")
    cfg, q, k, v, codes = workload(cfg_index)
    o = gpu_attention(q, k, v)
    assert not np.any(np.isnan(testkit.bf16_to_f32(o)))
    rows = sample_rows_strided(cfg.B, cfg.H, cfg.Nq, FULL_SIZE_STRIDE[cfg_index], seed=cfg_index)
    want, _, _ = oracle.attention_rows(codes, SCALE, rows)
    got = o[rows[:, 0], rows[:, 2], rows[:, 1]]
    check(got, want, v, f"{cfg.name}, {len(rows)} rows")


@pytest.mark.parametrize("N", [1, 2, 127, 128, 129, 255, 257, 600])
def test_ragged_self(device, N):
    log(f"attention tails N={N}")
    cfg = testkit.CONFIGS[4]
    q, k, v = testkit.make_inputs(cfg, seed=200 + N, H=3, Nq=N, Nkv=N)
    o = gpu_attention(q, k, v)
    check(o, oracle.attention(oracle.quantize(q, k, v), SCALE), v, f"N={N}")


@pytest.mark.parametrize("Nq,Nkv", [(300, 512), (1, 1000), (129, 1), (1000, 130), (64, 4608)])
def test_cross_shapes(device, Nq, Nkv):
    log(f"attention cross Nq={Nq} Nkv={Nkv}")
    cfg = testkit.CONFIGS[3]
    q, k, v = testkit.make_inputs(cfg, seed=11, B=2, H=3, Nq=Nq, Nkv=Nkv)
    o = gpu_attention(q, k, v)
    check(o, oracle.attention(oracle.quantize(q, k, v), SCALE), v, f"{Nq}x{Nkv}")


@pytest.mark.parametrize("cfg_index", [2, 4])
@pytest.mark.parametrize("scale", [0.01, 0.2, 0.5, 1.0])
def test_softmax_scales(device, cfg_index, scale):
    # scale 1.0 makes the logits ~11x sharper than the workloads' 1/sqrt(128);
    # the kernel is held to the same bar against the oracle there (three key
    # tiles per row, so the online softmax rescales)
    log(f"attention softmax_scale={scale}, workload {cfg_index} recipe")
    cfg = testkit.CONFIGS[cfg_index]
    q, k, v = testkit.make_inputs(cfg, seed=300 + cfg_index, H=2, Nq=384, Nkv=384)
    o = gpu_attention(q, k, v, scale)
    check(o, oracle.attention(oracle.quantize(q, k, v), scale), v, f"scale {scale}")


def test_sharp_softmax_against_exact_attention(device):
    # beside the oracle bar: at scale 1.0 the kernel is also no farther from
    # exact FP64 attention than the oracle (both are dominated by the INT8
    # score error there)
    log("attention softmax_scale=1.0 against the oracle and exact attention")
    cfg = testkit.CONFIGS[2]
    q, k, v = testkit.make_inputs(cfg, H=2, Nq=512, Nkv=512)
    ob = gpu_attention(q, k, v, 1.0)
    orb = oracle.attention(oracle.quantize(q, k, v), 1.0)
    check(ob, orb, v, "scale 1.0")
    o = testkit.bf16_to_f32(ob).astype(np.float64).ravel()
    orc = testkit.bf16_to_f32(orb).astype(np.float64).ravel()
    ref = oracle.bruteforce(q, k, v, 1.0).ravel()
    mv = maxv(v)
    cos = lambda a, b: float(a @ b / np.sqrt((a @ a) * (b @ b)))  # noqa: E731
    e_gpu, e_orc = np.abs(o - ref).max() / mv, np.abs(orc - ref).max() / mv
    log(f"  vs exact: kernel max err {e_gpu:.3e} cos {cos(o, ref):.6f}; oracle {e_orc:.3e} cos {cos(orc, ref):.6f}")
    assert cos(o, ref) >= cos(orc, ref) - 2e-4


def test_zero_q_matches_closed_form(device):
    log("attention Q = 0")
    cfg = testkit.CONFIGS[1]
    _, k, v = testkit.make_inputs(cfg, seed=9, Nq=130, Nkv=300)
    q = np.zeros((1, 130, 2, 128), np.uint16)
    o = gpu_attention(q, k, v)
    check(o, oracle.attention(oracle.quantize(q, k, v), SCALE), v, "Q = 0")


def test_zero_k_ragged(device):
    # every K block scale is 0, so every score is 0; the tail tile is masked
    log("attention K = 0, ragged")
    cfg = testkit.CONFIGS[1]
    q, _, v = testkit.make_inputs(cfg, seed=10, Nq=200, Nkv=333)
    k = np.zeros((1, 333, 2, 128), np.uint16)
    o = gpu_attention(q, k, v)
    check(o, oracle.attention(oracle.quantize(q, k, v), SCALE), v, "K = 0")


def test_single_key(device):
    log("attention Nkv = 1")
    cfg = testkit.CONFIGS[1]
    q, k, v = testkit.make_inputs(cfg, seed=13, Nq=70, Nkv=1)
    o = gpu_attention(q, k, v)
    want = oracle.attention(oracle.quantize(q, k, v), SCALE)
    assert np.array_equal(o, want)


def test_strided_output_and_3d(device):
    import torch
    log("attention strided output / 3D inputs")
    cfg = testkit.CONFIGS[2]
    q, k, v = testkit.make_inputs(cfg, H=4, Nq=384, Nkv=384)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    p = sattn.quantize_qkv(qd, kd, vd)
    ref = sattn.fwd(p)
    wide = torch.full((1, 384, 7, 128), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    out = wide[:, :, 2:6]
    sattn.fwd(p, out=out)
    assert torch.equal(out, ref)
    assert torch.isnan(wide[:, :, :2]).all() and torch.isnan(wide[:, :, 6:]).all()
    o3 = sattn.attention(qd[0], kd[0], vd[0])
    assert o3.shape == (384, 4, 128) and torch.equal(o3, ref[0])


def test_deterministic_and_fully_written(device):
    import torch
    log("attention determinism")
    cfg = testkit.CONFIGS[4]
    q, k, v = testkit.make_inputs(cfg, H=6, Nq=2000, Nkv=2000)
    p = sattn.quantize_qkv(to_dev(q), to_dev(k), to_dev(v))
    a = torch.full((1, 2000, 6, 128), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    sattn.fwd(p, out=a)
    b = sattn.fwd(p)
    torch.cuda.synchronize()
    assert not torch.isnan(a).any()
    assert torch.equal(a, b)


def test_device_errors_raise(device):
    import torch
    q = torch.zeros(1, 64, 2, 64, dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(NotImplementedError):
        sattn.quantize_qkv(q, q, q)
    q = torch.zeros(1, 64, 2, 128, dtype=torch.bfloat16, device="cuda:0")
    p = sattn.quantize_qkv(q, q, q)
    with pytest.raises(ValueError):
        sattn.fwd(p, softmax_scale=float("nan"))
    with pytest.raises(ValueError):
        sattn.fwd(p, out=torch.empty(1, 63, 2, 128, dtype=torch.bfloat16, device="cuda:0"))
