"""GPU parity of attention with many query tiles over short key sequences
(2 to 16 key tiles of 128): the regime of text cross-attention, where each
workgroup's output write is a large share of its work.  The BF16 rows go
out through LDS in whole 128-byte lines; these cases cover ragged Q and K
tails, tiles that cross heads in the launch order, strided outputs and the
16-tile sweep, with outputs and LSE against the oracle in both Q/K formats."""
import math

import numpy as np
import pytest

import oracle
import precision_flash_attention_amd as sattn
import testkit
from gpu_helpers import check_rows, from_dev, log, lse_bar, out_bar, sample_rows_strided, to_dev

pytestmark = pytest.mark.gpu
SCALE = 1.0 / math.sqrt(128.0)


def maxv(v):
    return float(np.abs(testkit.bf16_to_f32(v)).max())


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
@pytest.mark.parametrize("B,H,Nq,Nkv", [(1, 11, 16300, 300), (1, 8, 16384, 256), (2, 9, 7000, 77),
                                        (1, 300, 100, 200), (1, 290, 200, 512), (1, 8, 16384, 128),
                                        (1, 12, 9000, 384)])
def test_full_output_and_lse(device, fmt, B, H, Nq, Nkv):
    # (1, 11, 16300, 300): Q tail of 172 rows (the last 256-query tile's
    # second block holds 44), K tail of 44 keys; (1, 8, 16384, 256): exact;
    # (2, 9, 7000, 77): one key tile, 77 keys; (1, 300, 100, 200): one query
    # tile per head, its second Q block absent; (1, 290, 200, 512): one
    # ragged query tile per head against four full key tiles; (1, 8, 16384,
    # 128) and (1, 12, 9000, 384): one and three full key tiles.  Key counts
    # that are multiples of 128 run the instances without tail masking.
    q, k, v = testkit.make_inputs(testkit.CONFIGS[3], seed=31 + H, B=B, H=H, Nq=Nq, Nkv=Nkv)
    p = sattn.quantize_qkv(to_dev(q), to_dev(k), to_dev(v), qk_format=fmt)
    o, lse = sattn.fwd_cross(p, SCALE, return_lse=True)
    o = from_dev(o)
    lse = lse.cpu().numpy().astype(np.float64)
    c = oracle.quantize(q, k, v, qk_format=fmt)
    ref, ref_lse = oracle.attention(c, SCALE, return_lse=True)
    check_rows(o, ref, v, out_bar(c, SCALE), f"short-KV {B}x{H}x{Nq}x{Nkv} [{fmt}]")
    lw = np.max(np.abs(lse - ref_lse) / lse_bar(c, SCALE))
    log(f"    lse worst / bar {lw:.3f}")
    assert lw <= 1.0


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
def test_sixteen_key_tiles_sampled(device, fmt):
    B, H, Nq, Nkv = 2, 5, 13100, 2000     # 16 key tiles, tail of 80 keys
    q, k, v = testkit.make_inputs(testkit.CONFIGS[4], seed=41, B=B, H=H, Nq=Nq, Nkv=Nkv)
    p = sattn.quantize_qkv(to_dev(q), to_dev(k), to_dev(v), qk_format=fmt)
    o = from_dev(sattn.fwd_cross(p, SCALE))
    c = oracle.quantize(q, k, v, qk_format=fmt)
    rows = sample_rows_strided(B, H, Nq, 16, seed=42)
    ref, _, _ = oracle.attention_rows(c, SCALE, rows)
    check_rows(o[rows[:, 0], rows[:, 2], rows[:, 1]], ref, v, out_bar(c, SCALE, rows),
               f"short-KV 16 key tiles [{fmt}], {len(rows)} rows")


def test_strided_output_equals_contiguous(device):
    import torch
    B, H, Nq, Nkv = 2, 4, 16400, 400
    q, k, v = testkit.make_inputs(testkit.CONFIGS[3], seed=43, B=B, H=H, Nq=Nq, Nkv=Nkv)
    p = sattn.quantize_qkv(to_dev(q), to_dev(k), to_dev(v))
    o1 = sattn.fwd_cross(p, SCALE)
    big = torch.zeros(B, Nq, H, 256, dtype=torch.bfloat16, device="cuda:0")
    view = big[..., 64:192]
    o2 = sattn.fwd_cross(p, SCALE, out=view)
    assert o2.data_ptr() == view.data_ptr()
    assert torch.equal(o1, view)
    assert not big[..., :64].any() and not big[..., 192:].any()
    # and a repeat launch gives the same bits
    assert torch.equal(o1, sattn.fwd_cross(p, SCALE))
