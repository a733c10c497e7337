"""The longest sequences the library accepts: 2^24 tokens per head
(SATTN_MAX_SEQ), on the key side and on the query side.

At that length one head's BF16 tensor is 4 GiB and its codes 2 GiB, so every
byte offset of the quantize and attention kernels passes 2^31.  The oracle
cannot run the full problem in test time.  So the inputs are periodic, and
their full-size results follow from a one-period problem that the oracle
does run.
- Zero keys give every score 0, so each row's softmax is uniform over the
  keys.
- A tensor made of one 128-token block repeated 2^17 times has the same
  channel scales and, block by block, the same codes as that block alone.
- Its uniform average equals the average over one period.
So the full-size codes must be the one-period codes tiled, byte for byte.
The outputs must match the oracle's output of the one-period problem within
the parity bar, and the log-sum-exp is the one-period value plus ln(2^17).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import precision_flash_attention_amd as sattn
import testkit
from gpu_helpers import MAX_ERR, MIN_COS, assert_codes_equal, from_dev, log, parity, to_dev

pytestmark = pytest.mark.gpu

NMAX = 1 << 24          # SATTN_MAX_SEQ
PERIOD = 128
REPS = NMAX // PERIOD   # 2^17
SCALE = 1.0 / math.sqrt(128.0)
CFG = testkit.CONFIGS[3]


def _period_inputs(seed):
    """One 128-token block of Q and of V (the text cross-attention recipe)
    and 256 tokens of V, seeded."""
    q, _, v = testkit.make_inputs(CFG, seed=seed, B=1, H=1, Nq=PERIOD, Nkv=2 * PERIOD)
    return q, v


def _tiled(block_bits: np.ndarray) -> torch.Tensor:
    """[1, 128, 1, 128] BF16 bits -> the block repeated to [1, 2^24, 1, 128] on the device."""
    return to_dev(block_bits).repeat(1, REPS, 1, 1)


def _unpack_codes(p):
    """The canonical codes and scales of a packed buffer (host copy)."""
    return sattn.unpack_host(p)


def _check_max_err(o_gpu_bits, o_ref_bits, v_bits, what):
    err, c = parity(o_gpu_bits, o_ref_bits, float(np.abs(testkit.bf16_to_f32(v_bits)).max()))
    log(f"  {what}: max err / max|V| = {err:.3e}, cos = {c:.7f}")
    assert err <= MAX_ERR and c >= MIN_COS, (what, err, c)


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
def test_longest_key_sequence(device, fmt):
    log(f"max sizes ({fmt} Q/K): Nkv = 2^24 (K = 0, V = one 128-token block x {REPS}), Nq = 128")
    q, vb = _period_inputs(seed=31)
    v = np.ascontiguousarray(vb[:, :PERIOD])
    k0 = np.zeros_like(v)
    # one period, GPU and oracle
    small = sattn.quantize_qkv(to_dev(q), to_dev(k0), to_dev(v), qk_format=fmt)
    want = oracle.quantize(q, k0, v, qk_format=fmt)
    got_small = _unpack_codes(small)
    assert_codes_equal(got_small, want)
    o_ref, lse_ref = oracle.attention(want, SCALE, return_lse=True)
    # full length
    kd = torch.zeros((1, NMAX, 1, 128), dtype=torch.bfloat16, device=device)
    vd = _tiled(v)
    big = sattn.quantize_qkv(to_dev(q), kd, vd, qk_format=fmt)
    torch.cuda.synchronize()
    del kd, vd
    log("  quantized; unpacking")
    got = _unpack_codes(big)
    assert np.array_equal(got["q8"].view(np.uint8), got_small["q8"].view(np.uint8))
    assert np.array_equal(got["q_scale"].view(np.uint32), got_small["q_scale"].view(np.uint32))
    assert not got["k8"].any() and not got["k_scale"].any() and not got["k_mean"].any()
    assert np.array_equal(got["v_scale"].view(np.uint32), want["v_scale"].view(np.uint32))
    v8 = got["v8"].reshape(REPS, PERIOD, 128)
    bad = np.flatnonzero((v8 != want["v8"].reshape(1, PERIOD, 128)).any(axis=(1, 2)))
    assert bad.size == 0, f"V codes of {bad.size} periods differ, first {bad[:5].tolist()}"
    del got, v8
    for splits in (1, 0):
        log(f"  attention, num_splits={splits}")
        o, lse = sattn.fwd_cross(big, SCALE, return_lse=True, num_splits=splits)
        torch.cuda.synchronize()
        _check_max_err(from_dev(o), o_ref, v, f"Nkv = 2^24, num_splits={splits}")
        # ln(sum over 2^24 keys) = ln(sum over one period) + ln(2^17), all logits equal
        d = np.abs(lse.cpu().numpy().astype(np.float64) - (lse_ref + math.log(REPS))).max()
        log(f"  LSE: max |lse - (lse_period + ln 2^17)| = {d:.2e}")
        assert d <= 2e-5, d


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
def test_longest_query_sequence(device, fmt):
    log(f"max sizes ({fmt} Q/K): Nq = 2^24 (Q = one 128-token block x {REPS}), Nkv = 256 (K = 0)")
    q, v = _period_inputs(seed=32)
    k0 = np.zeros_like(v)
    small = sattn.quantize_qkv(to_dev(q), to_dev(k0), to_dev(v), qk_format=fmt)
    want = oracle.quantize(q, k0, v, qk_format=fmt)
    got_small = _unpack_codes(small)
    assert_codes_equal(got_small, want)
    o_ref = oracle.attention(want, SCALE)                    # [1, 128, 1, 128] BF16 bits
    qd = _tiled(q)
    big = sattn.quantize_qkv(qd, to_dev(k0), to_dev(v), qk_format=fmt)
    torch.cuda.synchronize()
    del qd
    log("  quantized; unpacking")
    got = _unpack_codes(big)
    q8 = got["q8"].view(np.uint8).reshape(REPS, PERIOD, 128)
    bad = np.flatnonzero((q8 != want["q8"].view(np.uint8).reshape(1, PERIOD, 128)).any(axis=(1, 2)))
    assert bad.size == 0, f"Q codes of {bad.size} periods differ, first {bad[:5].tolist()}"
    qs = got["q_scale"].reshape(-1).view(np.uint32)
    assert np.all(qs == want["q_scale"].reshape(-1).view(np.uint32)[0])
    for n in ("k8", "v8", "k_scale", "v_scale", "k_mean"):
        assert np.array_equal(got[n].view(np.uint8), want[n].view(np.uint8)), n
    del got, q8
    log("  attention")
    o = sattn.fwd_cross(big, SCALE)
    torch.cuda.synchronize()
    # every row against the one-period rows, on the device
    ref = to_dev(o_ref).float().reshape(1, PERIOD, 128)
    of = o.float().reshape(REPS, PERIOD, 128)
    maxv = float(np.abs(testkit.bf16_to_f32(v)).max())
    err = float((of - ref).abs().max()) / maxv
    f64 = torch.float64
    cos = float((of * ref).sum(dtype=f64)
                / torch.sqrt((of * of).sum(dtype=f64) * (ref * ref).sum(dtype=f64) * REPS))
    log(f"  Nq = 2^24: max err / max|V| = {err:.3e}, cos = {cos:.7f}")
    assert err <= MAX_ERR and cos >= MIN_COS, (err, cos)
    # and the first period's rows by the common metric
    _check_max_err(from_dev(o[:, :PERIOD]), o_ref, v, "Nq = 2^24, first period")
