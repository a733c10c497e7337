"""Exhaustive sweeps of the GPU quantizer's division shortcuts.

The kernels form x * fl(1/s) instead of the correctly rounded x / s and fall
back to the exact division only near a rounding boundary (INT8) or when the
two ends of the quotient's error interval encode differently (E4M3).  These
tests run every pair (x, amax) of finite BF16 values with |x| <= amax through
the real quantize entry point and compare codes and scales with the oracle:

- INT8 (Q path; K uses the same code): Q blocks of 128 tokens x 128 channels,
  each holding one amax value and a run of the BF16 values not above it, over
  all 32639 positive finite amax values: about 1.07e9 pairs.  The same blocks
  run through the FP8 Q/K format (E4M3 codes, block scale amax/448).
- E4M3 (V path): one channel per amax value (255 heads x 128 channels), its
  65536 tokens holding every BF16 value not above it in magnitude.

Both also cover every Q block scale amax/127 and every V channel scale
amax/448 the BF16 inputs can produce, subnormal scales included."""
import numpy as np
import pytest

import oracle
import precision_flash_attention_amd as sattn
from gpu_helpers import log

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

AMAX_BITS = np.arange(1, 0x7F80, dtype=np.int64)  # every positive finite BF16


def _values_up_to(a: int) -> np.ndarray:
    """Bit patterns of all BF16 x with |x| <= the BF16 value with bits a."""
    pos = np.arange(0, a + 1, dtype=np.uint16)
    neg = (np.arange(1, a + 1, dtype=np.uint32) | 0x8000).astype(np.uint16)
    return np.concatenate([pos, neg])


@pytest.mark.parametrize("qk_format", ["int8", "fp8"])
def test_q_codes_all_bf16_pairs(device, qk_format):
    import torch
    per = 128 * 128 - 1  # values per block besides its amax
    counts = (2 * AMAX_BITS + 1 + per - 1) // per
    nblk = int(counts.sum())
    log(f"{qk_format} Q sweep: {nblk} Q blocks, {int((2 * AMAX_BITS + 1).sum())} pairs")
    blocks = np.zeros((nblk, 128 * 128), np.uint16)
    i = 0
    for a, c in zip(AMAX_BITS.tolist(), counts.tolist()):
        vals = _values_up_to(a)
        pad = np.zeros(c * per, np.uint16)
        pad[: vals.size] = vals
        blocks[i:i + c, 0] = a
        blocks[i:i + c, 1:] = pad.reshape(c, per)
        i += c
    Nq = nblk * 128
    q = blocks.reshape(1, Nq, 1, 128)
    k = np.zeros((1, 1, 1, 128), np.uint16)
    v = np.zeros((1, 1, 1, 128), np.uint16)
    as_dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)  # noqa: E731
    got = sattn.unpack_host(sattn.quantize_qkv(as_dev(q), as_dev(k), as_dev(v), qk_format=qk_format))
    want = oracle.quantize(q, k, v, qk_format=qk_format)
    assert np.array_equal(got["q_scale"].view(np.uint32), want["q_scale"].view(np.uint32))
    bad = got["q8"] != want["q8"]
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{int(bad.sum())} {qk_format} codes differ, first at {idx.tolist()}")
    log(f"  {q.size} codes and {nblk} block scales equal the oracle")


def test_e4m3_codes_all_bf16_pairs(device):
    import torch
    H, N = 255, 65536
    C = H * 128
    log(f"E4M3 sweep: {C} channels x {N} tokens")
    cols = np.zeros((C, N), np.uint16)  # channel-major while filling
    amax = np.zeros(C, np.int64)
    amax[: AMAX_BITS.size] = AMAX_BITS
    amax[AMAX_BITS.size:] = 0x7F7F     # the one spare channel repeats the largest
    for c in range(C):
        vals = _values_up_to(int(amax[c]))
        cols[c, : vals.size] = vals     # the rest of the channel stays +0
    v = np.ascontiguousarray(cols.T).reshape(1, N, H, 128)
    del cols
    qd = torch.zeros((1, 1, H, 128), dtype=torch.bfloat16, device=device)
    kd = torch.zeros((1, N, H, 128), dtype=torch.bfloat16, device=device)
    vd = torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).to(device)
    got = sattn.unpack_host(sattn.quantize_qkv(qd, kd, vd))
    del qd, kd, vd
    torch.cuda.empty_cache()
    # the oracle's definition, channel by channel: s = fl(amax / 448) and
    # code = E4M3_RNE(clamp(fl(x / s), +-448)), with its arithmetic encoder
    amax_f = (amax.astype(np.uint32) << 16).view(np.float32)
    s = (amax_f / np.float32(448.0)).astype(np.float32)
    assert np.array_equal(got["v_scale"].reshape(C).view(np.uint32), s.view(np.uint32))
    v2 = v.reshape(N, C)
    g8 = got["v8"].reshape(H, N, 128)
    for h0 in range(0, H, 15):
        h1 = min(H, h0 + 15)
        x = (v2[:, h0 * 128:h1 * 128].astype(np.uint32) << 16).view(np.float32)
        y = np.clip(x / s[h0 * 128:h1 * 128], np.float32(-448.0), np.float32(448.0)).astype(np.float32)
        want = oracle.e4m3_encode(y)                               # [N, heads*128]
        have = g8[h0:h1].transpose(1, 0, 2).reshape(N, (h1 - h0) * 128)
        bad = have != want
        if bad.any():
            idx = np.argwhere(bad)[:5]
            raise AssertionError(f"heads {h0}..{h1}: {int(bad.sum())} E4M3 codes differ, first (token, ch) "
                                 f"{idx.tolist()}")
    log(f"  {v.size} codes and {C} channel scales equal the oracle's definition")
