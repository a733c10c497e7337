"""Pins of the oracle's log-sum-exp output.

The FA4 autotuning page ("Validation", and its summary of what the tuner
preserves) lists a float32 LSE beside the attention output, and split-KV
results merged with it.  The oracle returns, per query row,

    lse = m + ln(l) + (the logit shift that K smoothing removed),

the log-sum-exp of the row's logits before smoothing, so that it estimates
ln sum_j exp(softmax_scale * q . k_j) of the inputs.  Pinned here against
closed forms, exact FP64 log-sum-exp within a bound derived from the
quantizers' rounding, the merge rule over disjoint key sets, and the key
shift it must follow."""
import math

import numpy as np
import pytest

import oracle
import testkit

D = 128
SCALE = 1.0 / math.sqrt(128.0)


def f64(bits):
    return testkit.bf16_to_f32(bits).astype(np.float64)


def bf16_of(x):
    x = np.asarray(x, np.float64).astype(np.float32)
    u = x.view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def exact_lse(q, k, scale):
    """ln sum_j exp(scale q_i . k_j) in FP64 from the BF16 inputs: [B, H, Nq]."""
    qf, kf = f64(q), f64(k)
    B, Nq, H, _ = q.shape
    out = np.empty((B, H, Nq))
    for b in range(B):
        for h in range(H):
            s = scale * (qf[b, :, h] @ kf[b, :, h].T)
            m = s.max(axis=1, keepdims=True)
            out[b, h] = (m + np.log(np.exp(s - m).sum(axis=1, keepdims=True)))[:, 0]
    return out


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
@pytest.mark.parametrize("Nkv", [1, 127, 300])
def test_zero_q_gives_log_of_the_key_count(fmt, Nkv):
    # every logit is 0 (and so is the smoothing shift): lse = ln(Nkv) exactly
    cfg = testkit.CONFIGS[2]
    _, k, v = testkit.make_inputs(cfg, seed=1, H=2, Nq=3, Nkv=Nkv)
    q = np.zeros((1, 3, 2, D), np.uint16)
    _, lse = oracle.attention(oracle.quantize(q, k, v, qk_format=fmt), SCALE, return_lse=True)
    assert np.all(lse == math.log(Nkv))


def _rounding_bounds(x, s, fmt):
    """A priori bound on |dequantized code - x| per element, for values x
    (FP64, [..., N, 128]) coded with per-row scales s ([..., N])."""
    s = s[..., None]
    if fmt == "int8":
        return np.broadcast_to(0.5 * s, x.shape) * (1 + 2.0 ** -20)
    # E4M3: half a step, 2^-4 relative for normal codes, 2^-10 s below them
    return (np.abs(x) * 2.0 ** -4 + s * 2.0 ** -10) * (1 + 2.0 ** -20)


def _lse_error_bound(q, k, c, fmt, scale):
    """max_j over a bound on |logit_oracle(i, j) - logit_exact(i, j)|, per row:
    the logits differ by the rounding of Q, of K - mean, and of the FP32
    difference K - mean; ln-sum-exp is 1-Lipschitz in the max norm."""
    qf, kf = f64(q), f64(k)
    B, Nq, H, _ = q.shape
    Nkv = k.shape[1]
    out = np.empty((B, H, Nq))
    for b in range(B):
        for h in range(H):
            km = c["k_mean"][b, h].astype(np.float64)
            qs = c["q_scale"][b, h][np.arange(Nq) // 128].astype(np.float64)
            ks = c["k_scale"][b, h][np.arange(Nkv) // 128].astype(np.float64)
            qa = np.abs(qf[b, :, h])
            kp = kf[b, :, h] - km
            ka = np.abs(kp)
            eq = _rounding_bounds(qf[b, :, h], qs, fmt)
            ek = _rounding_bounds(kp, ks, fmt)
            bound = scale * (eq @ (ka + ek).T + (eq @ np.abs(km))[:, None] + qa @ ek.T
                             + 2.0 ** -23 * (qa @ ka.T))
            out[b, h] = bound.max(axis=1)
    return out + 1e-6


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
@pytest.mark.parametrize("cfg_index", [1, 2, 4])
def test_close_to_exact_log_sum_exp(fmt, cfg_index):
    cfg = testkit.CONFIGS[cfg_index]
    q, k, v = testkit.make_inputs(cfg, seed=30 + cfg_index, H=2, Nq=200, Nkv=300)
    c = oracle.quantize(q, k, v, qk_format=fmt)
    _, lse = oracle.attention(c, SCALE, return_lse=True)
    ref = exact_lse(q, k, SCALE)
    err = np.abs(lse - ref)
    bound = _lse_error_bound(q, k, c, fmt, SCALE)
    assert np.all(err <= bound)
    # the bound adds every rounding error with the same sign; they are
    # independent, so typical rows sit far inside it (0.3 to 4 % seen), where
    # a dropped smoothing shift or a base-2 logarithm would not
    assert np.median(err / bound) <= 0.1


def test_single_key_lse_is_its_logit():
    # one key: l = 1, and the smoothed key is 0, so lse is the shift term
    # alone; it must equal the exact logit up to the rounding of Q
    cfg = testkit.CONFIGS[2]
    q, k, v = testkit.make_inputs(cfg, seed=5, H=3, Nq=130, Nkv=1)
    for fmt in ("int8", "fp8"):
        c = oracle.quantize(q, k, v, qk_format=fmt)
        assert np.all(c["k8"] == 0)
        _, lse = oracle.attention(c, SCALE, return_lse=True)
        ref = exact_lse(q, k, SCALE)
        assert np.all(np.abs(lse - ref) <= _lse_error_bound(q, k, c, fmt, SCALE))
        assert np.abs(lse - ref).max() > 0  # the Q rounding is visible


def _key_slice(c, t0, t1):
    """The codes restricted to key blocks [t0, t1) (same means and scales)."""
    s = dict(c)
    s["k8"] = c["k8"][:, :, 128 * t0:128 * t1]
    s["v8"] = c["v8"][:, :, 128 * t0:128 * t1]
    s["k_scale"] = c["k_scale"][:, :, t0:t1]
    return s


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
def test_merge_rule_over_disjoint_key_blocks(fmt):
    # ln(e^a + e^b) of the two halves' lse equals the whole's: the row sums
    # add, and the smoothing shift is the same for both halves.  Each p is
    # rounded to FP32 against a different maximum in the parts and in the
    # whole, so each row sum is exact only to 2^-24 relative: 2e-7 > 2 * 2^-24.
    cfg = testkit.CONFIGS[4]
    q, k, v = testkit.make_inputs(cfg, seed=8, H=2, Nq=150, Nkv=700)
    c = oracle.quantize(q, k, v, qk_format=fmt)
    o_all, lse = oracle.attention(c, SCALE, return_lse=True)
    o_a, lse_a = oracle.attention(_key_slice(c, 0, 2), SCALE, return_lse=True)
    o_b, lse_b = oracle.attention(_key_slice(c, 2, 6), SCALE, return_lse=True)
    assert np.abs(np.logaddexp(lse_a, lse_b) - lse).max() <= 2e-7
    # the outputs merge with the same weights, up to the P rounding of
    # each part (each quantizes 448 p against its own maximum)
    wa = np.exp(lse_a - lse).transpose(0, 2, 1)[..., None]
    wb = np.exp(lse_b - lse).transpose(0, 2, 1)[..., None]
    merged = wa * f64(o_a) + wb * f64(o_b)
    assert np.abs(merged - f64(o_all)).max() <= 3e-2 * np.abs(f64(v)).max()


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
def test_key_shift_moves_lse_by_the_shift_logit(fmt):
    # adding a vector c to every key adds scale * q . c to every logit, so to
    # the lse; values on a 1/8 grid keep every BF16 value and FP32 sum exact,
    # so the smoothed keys (and codes) do not change and only the Q rounding
    # separates the oracle's shift from the exact one
    rng = np.random.default_rng(4)
    q = bf16_of(rng.integers(-16, 17, size=(1, 140, 2, D)) / 8.0)
    k0 = rng.integers(-16, 17, size=(1, 256, 2, D)) / 8.0
    cvec = rng.integers(-8, 9, size=(1, 1, 2, D)) * 1.0
    v = bf16_of(rng.normal(size=(1, 256, 2, D)))
    ka, kb = bf16_of(k0), bf16_of(k0 + cvec)
    ca = oracle.quantize(q, ka, v, qk_format=fmt)
    cb = oracle.quantize(q, kb, v, qk_format=fmt)
    assert np.array_equal(ca["k8"], cb["k8"])
    _, la = oracle.attention(ca, SCALE, return_lse=True)
    _, lb = oracle.attention(cb, SCALE, return_lse=True)
    qf = f64(q)
    want = SCALE * np.einsum("nhd,hd->hn", qf[0], cvec[0, 0])[None]
    qs = ca["q_scale"][0][:, np.arange(140) // 128].astype(np.float64)  # [H, Nq]
    eq = _rounding_bounds(qf[0].transpose(1, 0, 2), qs, fmt)            # [H, Nq, D]
    bound = SCALE * (eq @ np.abs(cvec[0, 0])[:, :, None])[..., 0] + 1e-6
    assert np.all(np.abs((lb - la) - want)[0] <= bound)
    assert np.abs(want).max() > 1.0


def test_rows_entry_matches_all_rows():
    cfg = testkit.CONFIGS[3]
    q, k, v = testkit.make_inputs(cfg, seed=2, B=2, H=2, Nq=70, Nkv=260)
    c = oracle.quantize(q, k, v)
    o, lse = oracle.attention(c, SCALE, return_lse=True)
    rows = np.array([[0, 0, 0], [1, 1, 69], [0, 1, 33], [1, 0, 5]], np.int64)
    o_r, m, l, lse_r = oracle.attention_rows(c, SCALE, rows, return_lse=True)
    assert np.array_equal(lse_r, lse[rows[:, 0], rows[:, 1], rows[:, 2]])
    assert np.array_equal(o_r, o[rows[:, 0], rows[:, 2], rows[:, 1]])
