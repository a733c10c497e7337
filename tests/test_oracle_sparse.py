"""Pins of the oracle's block-sparse attention.

The MHA v4 page's import listing names a block-attention-mask-to-ragged-LUT
conversion and a block-sparse attention reference, and the AITER bump page
measures sparse ("spargeattn", "distilled_sparse") pipelines.  Reading taken:
query i attends key j iff mask[b, h, i // 128, j // 128], 128-token blocks on
both sides (the quantization blocks); the method is unchanged on the allowed
keys (the quantizer does not see the mask); a row with no allowed key has
output 0 and LSE -inf.  Pinned against the dense oracle (all-ones masks,
single allowed blocks, complementary masks), exact FP64 block-sparse
attention, and the empty-row convention."""
import math

import numpy as np
import pytest

import oracle
import testkit

D = 128
SCALE = 1.0 / math.sqrt(128.0)


def f64(bits):
    return testkit.bf16_to_f32(bits).astype(np.float64)


def exact_sparse(q, k, v, mask, scale):
    """softmax over the allowed keys in FP64 from the BF16 inputs; 0 rows."""
    qf, kf, vf = f64(q), f64(k), f64(v)
    B, Nq, H, _ = q.shape
    Nkv = k.shape[1]
    out = np.zeros((B, Nq, H, D))
    for b in range(B):
        for h in range(H):
            allowed = mask[b, h][np.arange(Nq) // 128][:, np.arange(Nkv) // 128].astype(bool)
            s = scale * (qf[b, :, h] @ kf[b, :, h].T)
            s = np.where(allowed, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            ok = np.isfinite(m[:, 0])
            w = np.zeros_like(s)
            w[ok] = np.exp(s[ok] - m[ok])
            den = w.sum(axis=1, keepdims=True)
            out[b, ok, h] = (w[ok] @ vf[b, :, h]) / den[ok]
    return out


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
def test_all_ones_mask_is_the_dense_oracle(fmt):
    cfg = testkit.CONFIGS[4]
    q, k, v = testkit.make_inputs(cfg, seed=1, H=2, Nq=300, Nkv=400)
    c = oracle.quantize(q, k, v, qk_format=fmt)
    mask = np.ones((1, 2, 3, 4), np.uint8)
    o, lse = oracle.attention_sparse(c, SCALE, mask, return_lse=True)
    o_d, lse_d = oracle.attention(c, SCALE, return_lse=True)
    assert np.array_equal(o, o_d) and np.array_equal(lse, lse_d)


def _key_slice(c, t0, t1):
    s = dict(c)
    s["k8"] = c["k8"][:, :, 128 * t0:128 * t1]
    s["v8"] = c["v8"][:, :, 128 * t0:128 * t1]
    s["k_scale"] = c["k_scale"][:, :, t0:t1]
    return s


@pytest.mark.parametrize("kb", [0, 1, 3])
def test_one_allowed_block_is_dense_attention_on_it(kb):
    # the same arithmetic on the same keys: bit-equal to the dense oracle
    # given only that block's codes (block 3 is the 44-key tail)
    cfg = testkit.CONFIGS[2]
    q, k, v = testkit.make_inputs(cfg, seed=2, H=2, Nq=200, Nkv=428)
    c = oracle.quantize(q, k, v)
    mask = np.zeros((1, 2, 2, 4), np.uint8)
    mask[..., kb] = 1
    o, lse = oracle.attention_sparse(c, SCALE, mask, return_lse=True)
    o_s, lse_s = oracle.attention(_key_slice(c, kb, kb + 1), SCALE, return_lse=True)
    assert np.array_equal(o, o_s) and np.array_equal(lse, lse_s)


def test_rows_without_keys_are_zero():
    cfg = testkit.CONFIGS[1]
    q, k, v = testkit.make_inputs(cfg, seed=3, Nq=300, Nkv=260)
    c = oracle.quantize(q, k, v)
    mask = np.ones((1, 2, 3, 3), np.uint8)
    mask[0, 1, 1] = 0          # head 1, queries 128..255: nothing allowed
    mask[0, 0, 2, 1:] = 0      # head 0, queries 256..299: only block 0
    o, lse = oracle.attention_sparse(c, SCALE, mask, return_lse=True)
    assert np.all(o[0, 128:256, 1] == 0) and np.all(lse[0, 1, 128:256] == -np.inf)
    assert np.all(np.isfinite(lse[0, 0])) and np.any(o[0, 256:, 0] != 0)
    o_d = oracle.attention(c, SCALE)
    assert np.array_equal(o[0, :128], o_d[0, :128])


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
@pytest.mark.parametrize("density", [0.2, 0.6])
def test_close_to_exact_block_sparse_attention(fmt, density):
    cfg = testkit.CONFIGS[2]
    q, k, v = testkit.make_inputs(cfg, seed=4, H=3, Nq=500, Nkv=700)
    mask = testkit.block_mask(1, 3, 500, 700, density, seed=9)
    mask[0, 0, 1] = 0  # one empty query block
    c = oracle.quantize(q, k, v, qk_format=fmt)
    o = f64(oracle.attention_sparse(c, SCALE, mask))
    ref = exact_sparse(q, k, v, mask, SCALE)
    a, b = o.ravel(), ref.ravel()
    assert float(a @ b / np.sqrt((a @ a) * (b @ b))) >= 0.99
    assert np.all(o[0, 128:256, 0] == 0) and np.all(ref[0, 128:256, 0] == 0)
    # the mask matters: dense attention is far from it
    dense = f64(oracle.attention(c, SCALE))
    assert np.abs(dense - ref).max() > 10 * np.abs(o - ref).max()


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
def test_complementary_masks_merge_to_dense(fmt):
    # the allowed and the forbidden keys of each row split its row sum
    cfg = testkit.CONFIGS[4]
    q, k, v = testkit.make_inputs(cfg, seed=5, H=2, Nq=260, Nkv=600)
    c = oracle.quantize(q, k, v, qk_format=fmt)
    mask = testkit.block_mask(1, 2, 260, 600, 0.5, seed=10, keep_diagonal=False)
    mask[..., 0] = 1   # every row keeps a block on each side
    mask[..., 1] = 0
    _, la = oracle.attention_sparse(c, SCALE, mask, return_lse=True)
    _, lb = oracle.attention_sparse(c, SCALE, 1 - mask, return_lse=True)
    _, ld = oracle.attention(c, SCALE, return_lse=True)
    assert np.abs(np.logaddexp(la, lb) - ld).max() <= 2e-7


def test_block_mask_generator():
    m = testkit.block_mask(2, 3, 1000, 3000, 0.3, seed=7)
    assert m.shape == (2, 3, 8, 24) and m.dtype == np.uint8
    assert np.array_equal(m, testkit.block_mask(2, 3, 1000, 3000, 0.3, seed=7))
    assert np.all(m[:, :, np.arange(8), np.arange(8)] == 1)
    assert 0.25 < m.mean() < 0.4


def test_rows_entry_matches_all_rows():
    cfg = testkit.CONFIGS[3]
    q, k, v = testkit.make_inputs(cfg, seed=6, B=2, H=2, Nq=300, Nkv=500)
    c = oracle.quantize(q, k, v)
    mask = testkit.block_mask(2, 2, 300, 500, 0.4, seed=11)
    mask[1, 0, 2] = 0
    o, lse = oracle.attention_sparse(c, SCALE, mask, return_lse=True)
    rows = np.array([[0, 0, 0], [1, 1, 299], [1, 0, 260], [0, 1, 140]], np.int64)
    o_r, _, _, lse_r = oracle.attention_rows(c, SCALE, rows, return_lse=True, block_mask=mask)
    assert np.array_equal(lse_r, lse[rows[:, 0], rows[:, 1], rows[:, 2]])
    assert np.array_equal(o_r, o[rows[:, 0], rows[:, 2], rows[:, 1]])
    assert lse_r[2] == -np.inf
