"""Pins of the oracle's quantizers against hand-computed cases.

Definitions (the method): Q/K per (batch, head, 128-token block) scale
amax/127 in FP32, round-half-even, clamp +-127; K mean-smoothed over the
sequence first (block sums in token order, then the sums in block order, one
division by Nkv); V per (batch, head, channel) scale amax/448 and OCP E4M3
round-to-nearest-even.  Every expected value below is worked out by hand in
the comment next to it.
"""
import numpy as np

import oracle
import testkit

D = 128


def bf16(x):
    """Exact BF16 bits of values that are representable in BF16."""
    f = np.asarray(x, dtype=np.float32)
    bits = f.view(np.uint32)
    assert np.all((bits & 0xFFFF) == 0), "value not exactly representable in BF16"
    return (bits >> 16).astype(np.uint16)


def zeros(B, N, H):
    return np.zeros((B, N, H, D), np.uint16)


def test_q_codes_round_half_even_at_unit_scale():
    # amax = 127 -> scale = 127/127 = 1 exactly, so the code is RNE(x)
    vals = [127.0, 2.5, 3.5, -2.5, 126.5, -126.5, 0.5, 1.5, -0.5, 0.25, 100.0, -127.0]
    want = [127, 2, 4, -2, 126, -126, 0, 2, 0, 0, 100, -127]
    q = zeros(1, 128, 1)
    q[0, : len(vals), 0, 0] = bf16(vals)
    c = oracle.quantize(q, zeros(1, 128, 1), zeros(1, 128, 1))
    assert c["q_scale"][0, 0, 0] == 1.0
    assert c["q8"][0, 0, : len(vals), 0].tolist() == want
    assert np.all(c["q8"][0, 0, len(vals):] == 0)


def test_q_scale_per_block_and_zero_block():
    # block 0 amax 254 -> scale 2; block 1 all zero -> scale 0, codes 0;
    # block 2 (tail of 44 tokens) amax 0.5 -> scale 0.5/127
    q = zeros(1, 300, 1)
    q[0, 5, 0, 3] = bf16(254.0)
    q[0, 6, 0, 4] = bf16(-3.0)      # -3/2 = -1.5 -> RNE -2
    q[0, 299, 0, 7] = bf16(0.5)     # 0.5 / fl(0.5/127) = 127 -> 127
    c = oracle.quantize(q, zeros(1, 300, 1), zeros(1, 300, 1))
    s = c["q_scale"][0, 0]
    assert s[0] == 2.0 and s[1] == 0.0
    assert s[2] == np.float32(0.5) / np.float32(127.0)
    assert c["q8"][0, 0, 5, 3] == 127 and c["q8"][0, 0, 6, 4] == -2
    assert np.all(c["q8"][0, 0, 128:256] == 0)
    assert c["q8"][0, 0, 299, 7] == 127


def test_k_mean_uses_block_then_sequential_fp32_order():
    # block 0: 2^24 then 127 ones; each +1 is a tie at ulp 2 and rounds back
    # to 2^24, so the block sum is 2^24.  block 1: 128 ones -> 128.
    # total 2^24 + 128 = 16777344 (exact), mean = 16777344 / 256 = 65536.5.
    # (An exact or pairwise sum would give (2^24 + 255) / 256 = 65536.996...)
    k = zeros(1, 256, 1)
    k[0, :, 0, 0] = bf16([1.0])
    k[0, 0, 0, 0] = bf16(2.0 ** 24)
    c = oracle.quantize(zeros(1, 256, 1), k, zeros(1, 256, 1))
    assert c["k_mean"][0, 0, 0] == 65536.5
    assert c["k_mean"][0, 0, 1] == 0.0


def test_k_smoothing_removes_the_shared_bias_exactly():
    # k[n, d] = bias_d + (+1 or -1 alternating): mean = bias_d exactly,
    # k' = +-1, block amax 1 -> scale 1/127, codes +-127.
    N = 256
    bias = np.array([3.0, -40.0, 0.0, 96.0] + [7.0] * (D - 4), np.float32)
    sign = np.where(np.arange(N) % 2 == 0, 1.0, -1.0).astype(np.float32)
    k = zeros(1, N, 1)
    k[0, :, 0, :] = bf16(bias[None, :] + sign[:, None])
    c = oracle.quantize(zeros(1, N, 1), k, zeros(1, N, 1))
    assert np.array_equal(c["k_mean"][0, 0], bias)
    assert np.all(c["k_scale"][0, 0] == np.float32(1.0) / np.float32(127.0))
    assert np.array_equal(c["k8"][0, 0, :, 0], (127 * sign).astype(np.int8))


def test_k_tail_tokens_do_not_enter_mean_or_amax():
    # Nkv = 129: one token in block 1.  All tokens 2.0 except the last, 6.0:
    # sum = 128*2 + 6 = 262, mean = 262/129 = fl32(2.031007...)
    k = zeros(1, 129, 1)
    k[0, :, 0, :] = bf16([2.0])
    k[0, 128, 0, :] = bf16([6.0])
    c = oracle.quantize(zeros(1, 129, 1), k, zeros(1, 129, 1))
    mean = np.float32(262.0) / np.float32(129.0)
    assert c["k_mean"][0, 0, 0] == mean
    # block 1 holds the single token: k' = 6 - mean, its own amax -> code 127
    assert c["k8"][0, 0, 128, 0] == 127
    assert c["k_scale"][0, 0, 1] == (np.float32(6.0) - mean) / np.float32(127.0)


def test_v_codes_at_unit_scale():
    # channel amax 448 -> scale 1 -> codes are the E4M3 codes of the values
    v = zeros(1, 8, 1)
    v[0, :, 0, 0] = bf16([448.0, 1.0, -0.5, 2.0 ** -9, 2.0 ** -10, 1.0625, 240.0, -448.0])
    c = oracle.quantize(zeros(1, 8, 1), zeros(1, 8, 1), v)
    assert c["v_scale"][0, 0, 0] == 1.0
    assert c["v8"][0, 0, :, 0].tolist() == [0x7E, 0x38, 0xB0, 0x01, 0x00, 0x38, 0x77, 0xFE]
    # all-zero channel: scale 0, codes 0x00
    assert c["v_scale"][0, 0, 1] == 0.0 and np.all(c["v8"][0, 0, :, 1] == 0)


def test_v_scale_power_of_two():
    # amax 7 -> scale 7/448 = 1/64 exactly; v = 3.5 -> 224 -> code 0x76
    v = zeros(1, 3, 1)
    v[0, :, 0, 5] = bf16([7.0, 3.5, -0.0078125])   # last: -0.5 -> 0xB0
    c = oracle.quantize(zeros(1, 3, 1), zeros(1, 3, 1), v)
    assert c["v_scale"][0, 0, 5] == 2.0 ** -6
    assert c["v8"][0, 0, :, 5].tolist() == [0x7E, 0x76, 0xB0]


def test_subnormal_block_is_exact():
    # q = 2^-130 (BF16 subnormal).  2^-130/127 lies in the FP32 subnormal
    # range with quantum 2^-149: 2^19/127 = 4128.25 -> s = 4128 * 2^-149;
    # x/s = 2^19/4128 = 127.0078 -> code 127.
    q = zeros(1, 128, 1)
    q[0, 0, 0, 0] = np.uint16(0x0008)  # 2^-130 = 8 * 2^-133, BF16 subnormal bits 0x0008
    assert testkit.bf16_to_f32(q[0, 0, 0, :1])[0] == np.float32(2.0 ** -130)
    c = oracle.quantize(q, zeros(1, 128, 1), zeros(1, 128, 1))
    assert c["q_scale"][0, 0, 0] == np.float32(4128 * 2.0 ** -149)
    assert c["q8"][0, 0, 0, 0] == 127


def test_codes_never_minus_128_and_bounded():
    cfg = testkit.CONFIGS[4]
    q, k, v = testkit.make_inputs(cfg, H=2, Nq=300, Nkv=300)
    c = oracle.quantize(q, k, v)
    for name in ("q8", "k8"):
        assert c[name].min() >= -127 and c[name].max() <= 127
        # each block's amax element maps to +-127
        B, H, N, _ = c[name].shape
        for t in range((N + 127) // 128):
            blk = np.abs(c[name][0, 0, 128 * t: 128 * (t + 1)].astype(np.int32))
            assert blk.max() == 127
    assert not np.any((c["v8"] & 0x7F) == 0x7F), "no NaN codes"
    # each channel's amax element maps to +-448
    assert np.all(np.max(c["v8"][0, 0] & 0x7F, axis=0) == 0x7E)
