"""GPU parity of block-sparse attention (the MHA v4 page's block-mask-to-
ragged-LUT conversion and block-sparse reference) against
``oracle.attention_sparse``: the table is exact index work (bit-exact
against its definition), an all-ones mask reproduces the dense FP8 Q/K kernel
bit for bit in both Q/K formats, and outputs and LSE meet the dense bars on
the allowed keys."""
import math

import numpy as np
import pytest

import oracle
import precision_flash_attention_amd as sattn
import testkit
from gpu_helpers import (MIN_COS, from_dev, log, lse_bar, out_bar, parity, row_errors, sample_rows_strided,
                         to_dev)

pytestmark = pytest.mark.gpu
SCALE = 1.0 / math.sqrt(128.0)


def maxv(v):
    return float(np.abs(testkit.bf16_to_f32(v)).max())


def mask_dev(mask):
    import torch
    return torch.from_numpy(np.ascontiguousarray(mask)).to("cuda:0")


def expected_table(mask):
    """Per 256-query tile g = (b*H + h)*mt + m: the ascending key blocks that
    query block 2m or 2m+1 attends, with bit 30 / bit 31 marking which."""
    B, H, nbq, nbk = mask.shape
    mt = (nbq + 1) // 2
    counts, entries = [], []
    for b in range(B):
        for h in range(H):
            for m in range(mt):
                a0 = mask[b, h, 2 * m] != 0
                a1 = mask[b, h, 2 * m + 1] != 0 if 2 * m + 1 < nbq else np.zeros(nbk, bool)
                kbs = np.nonzero(a0 | a1)[0]
                counts.append(len(kbs))
                entries.append([int(k) | (int(a0[k]) << 30) | (int(a1[k]) << 31) for k in kbs])
    return np.array(counts, np.int32), entries


@pytest.mark.parametrize("shape", [(1, 2, 300, 700), (2, 3, 1000, 5000), (1, 1, 1, 1), (1, 2, 128, 8192 + 5)])
@pytest.mark.parametrize("density", [0.0, 0.3, 1.0])
def test_table_matches_its_definition(device, shape, density):
    B, H, Nq, Nkv = shape
    mask = testkit.block_mask(B, H, Nq, Nkv, density, seed=3, keep_diagonal=density > 0)
    lut = sattn.block_lut(mask_dev(mask), Nq, Nkv)
    raw = lut.buf.cpu().numpy()
    G = B * H * ((Nq + 255) // 256)
    nbk = (Nkv + 127) // 128
    cbytes = (G * 4 + 255) // 256 * 256
    counts = raw[:G * 4].view(np.int32)
    ent = raw[cbytes:cbytes + G * nbk * 4].view(np.uint32).reshape(G, nbk)
    want_c, want_e = expected_table(mask)
    assert np.array_equal(counts, want_c)
    for g in range(G):
        assert np.array_equal(ent[g, :counts[g]], np.array(want_e[g], np.uint32)), g


def run_sparse(q, k, v, mask, fmt="int8"):
    p = sattn.quantize_qkv(to_dev(q), to_dev(k), to_dev(v), qk_format=fmt)
    lut = sattn.block_lut(mask_dev(mask), p.Nq, p.Nkv)
    o, lse = sattn.fwd_sparse(p, lut, SCALE, return_lse=True)
    return from_dev(o), lse.cpu().numpy().astype(np.float64), p


def check(q, k, v, mask, fmt, what):
    o, lse, _ = run_sparse(q, k, v, mask, fmt)
    c = oracle.quantize(q, k, v, qk_format=fmt)
    ref, ref_lse = oracle.attention_sparse(c, SCALE, mask, return_lse=True)
    err, cs = parity(o, ref, maxv(v))
    ratio = float(np.max(row_errors(o, ref, maxv(v)) / out_bar(c, SCALE)))
    empty = ~np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(lse), ~empty), "rows without keys must be -inf, the rest finite"
    lerr = np.abs(np.where(empty, 0.0, lse) - np.where(empty, 0.0, ref_lse))
    lbar = lse_bar(c, SCALE)
    log(f"  {what} [{fmt}] density {mask.mean():.2f}: out err {err:.3e} (worst / bar {ratio:.3f}) "
        f"cos {cs:.7f}; lse worst / bar {np.max(lerr / lbar):.3f}; empty rows {int(empty.sum())}")
    assert ratio <= 1.0 and cs >= MIN_COS, (ratio, cs)
    assert np.all(lerr <= lbar)
    assert np.all(o[np.transpose(empty, (0, 2, 1))] == 0)


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
def test_all_ones_mask_is_the_dense_kernel(device, fmt):
    # the same tiles in the same order through the same arithmetic
    import torch
    cfg = testkit.CONFIGS[4]
    q, k, v = testkit.make_inputs(cfg, seed=40, H=3, Nq=700, Nkv=900)
    mask = np.ones((1, 3, 6, 8), np.uint8)
    o, lse, p = run_sparse(q, k, v, mask, fmt)
    od, lsed = sattn.fwd_cross(p, SCALE, return_lse=True)
    assert np.array_equal(o, from_dev(od))
    assert torch.equal(torch.from_numpy(lse).float(), lsed.cpu())


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
@pytest.mark.parametrize("density", [0.2, 0.6])
@pytest.mark.parametrize("shape", [(1, 3, 700, 900), (2, 2, 300, 1300)])
def test_random_masks(device, fmt, density, shape):
    B, H, Nq, Nkv = shape
    cfg = testkit.CONFIGS[4]
    q, k, v = testkit.make_inputs(cfg, seed=41, B=B, H=H, Nq=Nq, Nkv=Nkv)
    mask = testkit.block_mask(B, H, Nq, Nkv, density, seed=12)
    mask[0, 0, 1] = 0               # a query block without keys (the second of its tile)
    mask[-1, -1, 0] = 0             # and a first one
    mask[0, 1, 2, :] = 0
    mask[0, 1, 2, -1] = 1           # only the ragged tail block
    check(q, k, v, mask, fmt, f"{Nq}x{Nkv}")


def test_empty_mask(device):
    cfg = testkit.CONFIGS[2]
    q, k, v = testkit.make_inputs(cfg, seed=42, H=2, Nq=300, Nkv=500)
    mask = np.zeros((1, 2, 3, 4), np.uint8)
    o, lse, _ = run_sparse(q, k, v, mask)
    assert np.all(o == 0) and np.all(lse == -np.inf)


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
def test_wan_shape_half_density_sampled(device, fmt):
    cfg = testkit.CONFIGS[4]
    q, k, v = testkit.make_inputs(cfg)
    mask = testkit.block_mask(1, 40, cfg.Nq, cfg.Nkv, 0.5, seed=7)
    o, lse, _ = run_sparse(q, k, v, mask, fmt)
    c = oracle.quantize(q, k, v, qk_format=fmt)
    rows = sample_rows_strided(1, 40, cfg.Nq, 128, seed=13)
    ref, _, _, ref_lse = oracle.attention_rows(c, SCALE, rows, return_lse=True, block_mask=mask)
    got = o[rows[:, 0], rows[:, 2], rows[:, 1]]
    err, cs = parity(got, ref, maxv(v))
    ratio = float(np.max(row_errors(got, ref, maxv(v)) / out_bar(c, SCALE, rows)))
    lerr = np.abs(lse[rows[:, 0], rows[:, 1], rows[:, 2]] - ref_lse)
    lbar = lse_bar(c, SCALE, rows)
    log(f"  wan half-density [{fmt}], {len(rows)} rows: out err {err:.3e} (worst / bar {ratio:.3f}) "
        f"cos {cs:.7f}; lse worst / bar {np.max(lerr / lbar):.3f}")
    assert ratio <= 1.0 and cs >= MIN_COS
    assert np.all(lerr <= lbar)


def test_table_shape_mismatch_raises(device):
    import torch
    cfg = testkit.CONFIGS[1]
    q, k, v = testkit.make_inputs(cfg, Nq=300, Nkv=300)
    p = sattn.quantize_qkv(to_dev(q), to_dev(k), to_dev(v))
    with pytest.raises(ValueError):
        sattn.block_lut(torch.ones(1, 2, 2, 3, dtype=torch.uint8, device="cuda:0"), 300, 300)
    lut = sattn.block_lut(torch.ones(1, 2, 3, 2, dtype=torch.uint8, device="cuda:0"), 300, 200)
    with pytest.raises(ValueError):
        sattn.fwd_sparse(p, lut, SCALE)
