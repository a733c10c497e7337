"""Pins of the oracle's FP8 Q/K format (the FP8/FP8/BF16 row of the MHA v4
page's MI355X throughput table): Q and mean-smoothed K as OCP E4M3 with a
per-128-token-block scale amax/448, scores from exact dot products of the
decoded codes, and the rest of the method unchanged."""
import numpy as np
import pytest

import oracle
import testkit

D = 128
SCALE = 1.0 / np.sqrt(128.0)


def f32(bits):
    return testkit.bf16_to_f32(bits).astype(np.float64)


def bf16_of(x):
    x = np.asarray(x, np.float64).astype(np.float32)
    return ((x.view(np.uint32) + 0x7FFF + ((x.view(np.uint32) >> 16) & 1)) >> 16).astype(np.uint16)


def cos(a, b):
    a = a.ravel().astype(np.float64)
    b = b.ravel().astype(np.float64)
    return float(a @ b / np.sqrt((a @ a) * (b @ b)))


def run(q, k, v, scale=SCALE):
    c = oracle.quantize(q, k, v, qk_format="fp8")
    return f32(oracle.attention(c, scale)), c


def test_q_codes_follow_the_independent_nearest_encoder():
    # block 0: amax 448 -> scale exactly 1, codes are E4M3 of the values;
    # block 1: amax 224 -> scale 0.5, codes are E4M3 of twice the values.
    # Each is checked against the brute-force nearest-code encoder.
    rng = np.random.default_rng(1)
    q = np.zeros((1, 256, 1, D), np.float64)
    q[0, :128, 0] = rng.uniform(-448, 448, size=(128, D))
    q[0, 0, 0, 0] = 448.0
    q[0, 128:, 0] = rng.uniform(-224, 224, size=(128, D))
    q[0, 128, 0, 0] = -224.0
    qb = bf16_of(q)
    k = np.zeros((1, 1, 1, D), np.uint16)
    c = oracle.quantize(qb, k, k, qk_format="fp8")
    assert c["q_scale"][0, 0].tolist() == [1.0, 0.5]
    x = f32(qb)[0, :, 0]
    want = np.array([[oracle.e4m3_encode_nearest(x[n, d] / (1.0 if n < 128 else 0.5)) for d in range(D)]
                     for n in range(256)], np.uint8)
    assert np.array_equal(c["q8"][0, 0].view(np.uint8), want)
    # and every code decodes back within half an E4M3 step
    dec = oracle.e4m3_decode(c["q8"][0, 0].view(np.uint8)) * np.where(np.arange(256) < 128, 1.0, 0.5)[:, None]
    assert np.all(np.abs(dec - x) <= np.abs(x) * 2.0 ** -4 + 2.0 ** -10)


def test_zero_block_and_tail_rows():
    # an all-zero block has scale 0 and codes 0x00; the tail tokens of a
    # ragged block do not enter its amax
    cfg = testkit.CONFIGS[1]
    q, k, v = testkit.make_inputs(cfg, seed=4, Nq=300, Nkv=130)
    q[:, 128:256] = 0
    c = oracle.quantize(q, k, v, qk_format="fp8")
    assert np.all(c["q_scale"][:, :, 1] == 0.0)
    assert np.all(c["q8"][:, :, 128:256] == 0)
    amax_tail = np.abs(f32(q[:, 256:300])).max(axis=(1, 3))  # [B, H]
    assert np.array_equal(c["q_scale"][:, :, 2], (amax_tail.astype(np.float32) / np.float32(448.0)))


def test_k_smoothing_removes_a_shared_bias_exactly():
    # K on a coarse grid plus a per-channel bias: every FP32 sum is exact, the
    # mean equals the bias plus the grid's mean, so the codes equal those of
    # the unbiased K (whose mean is subtracted the same way)
    # (values on a 1/8 grid within +-10: exact in BF16, and all sums exact)
    rng = np.random.default_rng(2)
    grid = rng.integers(-16, 17, size=(1, 256, 1, D)) / 8.0
    bias = rng.integers(-8, 9, size=(1, 1, 1, D)) * 1.0
    q = bf16_of(rng.normal(size=(1, 128, 1, D)))
    k0, k1 = bf16_of(grid), bf16_of(grid + bias)
    c0 = oracle.quantize(q, k0, k0, qk_format="fp8")
    c1 = oracle.quantize(q, k1, k1, qk_format="fp8")
    assert np.array_equal(c0["k8"], c1["k8"])
    assert np.array_equal(c0["k_scale"], c1["k_scale"])


@pytest.mark.parametrize("N", [1, 7, 128, 129, 300])
def test_close_to_exact_attention(N):
    cfg = testkit.CONFIGS[1]
    q, k, v = testkit.make_inputs(cfg, seed=70 + N, Nq=N, Nkv=N)
    o, _ = run(q, k, v)
    ref = oracle.bruteforce(q, k, v, SCALE)
    assert cos(o, ref) >= 0.99
    assert np.abs(o - ref).max() <= 0.1


@pytest.mark.parametrize("cfg_index", [2, 4, 5])
def test_close_to_exact_attention_on_workload_recipes(cfg_index):
    cfg = testkit.CONFIGS[cfg_index]
    q, k, v = testkit.make_inputs(cfg, H=2, Nq=256, Nkv=384)
    o, _ = run(q, k, v)
    assert cos(o, oracle.bruteforce(q, k, v, SCALE)) >= 0.99


def test_key_shift_invariance():
    # exact in real arithmetic; here the shifted keys are re-rounded to BF16
    # (an input change of up to 2^-9 relative at |k + c| ~ 3..10) and their
    # smoothed values re-quantised with E4M3's 2^-4 relative step, so the
    # bound is looser than the INT8 format's.  Dropping the smoothing would
    # quantise |c| ~ 3 with that step and fall far below it.
    cfg = testkit.CONFIGS[1]
    q, k, v = testkit.make_inputs(cfg, seed=3, Nq=256, Nkv=256)
    c = np.random.default_rng(0).normal(0, 3.0, size=(1, 1, 2, D))
    o1, _ = run(q, k, v)
    o2, _ = run(q, bf16_of(f32(k) + c), v)
    assert cos(o1, o2) >= 0.999
    assert np.abs(o1 - o2).max() <= 4e-2 * np.abs(f32(v)).max()


def test_zero_q_is_exact_mean_of_dequantized_v():
    cfg = testkit.CONFIGS[1]
    _, k, v = testkit.make_inputs(cfg, seed=9, Nq=1, Nkv=300)
    q = np.zeros((1, 1, 2, D), np.uint16)
    o, c = run(q, k, v)
    num = oracle.e4m3_decode(c["v8"]).sum(axis=2)
    want = f32(bf16_of(num * c["v_scale"].astype(np.float64) / 300.0))
    assert np.array_equal(o[0, 0], want[0])


def test_dominant_key_selects_its_row():
    # one key aligned with the query and much larger than the rest
    cfg = testkit.CONFIGS[1]
    q, k, v = testkit.make_inputs(cfg, seed=21, Nq=1, Nkv=200)
    kf = f32(k) * 0.05
    kf[0, 77] = f32(q)[0, 0] * 4.0
    o, _ = run(q, bf16_of(kf), v, scale=1.0)
    assert np.abs(o[0, 0] - f32(v)[0, 77]).max() <= 0.05 * np.abs(f32(v)[0, 77]).max()
