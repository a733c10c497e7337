"""The device FP32 -> OCP E4M3 conversion of the V quantizer against the
oracle's encoder, on every FP32 bit pattern with |x| <= 448."""
import numpy as np
import pytest

import oracle
import precision_flash_attention_amd as sattn
from gpu_helpers import log

pytestmark = pytest.mark.gpu

LIMIT = 0x43E00000  # bit pattern of 448.0


@pytest.mark.parametrize("sign", [0, 1])
def test_exhaustive_against_oracle(device, sign):
    import torch
    chunk = 1 << 27
    base = sign << 31
    lo = 0
    while lo <= LIMIT:
        n = min(chunk, LIMIT + 1 - lo)
        bits = torch.arange(lo, lo + n, dtype=torch.int64, device="cuda:0") | base
        x = bits.to(torch.int32).view(torch.float32) if sign == 0 else \
            (bits - (1 << 32)).to(torch.int32).view(torch.float32)
        got = sattn.e4m3_encode(x).cpu().numpy()
        want = oracle.e4m3_encode_bits(base | lo, n)
        if not np.array_equal(got, want):
            i = int(np.argmax(got != want))
            raise AssertionError(f"pattern {base | (lo + i):#010x}: got {got[i]:#04x} want {want[i]:#04x}")
        lo += n
    log(f"  sign {sign}: {LIMIT + 1} patterns agree")


def test_clamps_beyond_448(device):
    import torch
    x = torch.tensor([449.0, 464.0, 500.0, 1e30, float("inf"), -500.0, -float("inf")],
                     device="cuda:0")
    assert sattn.e4m3_encode(x).cpu().tolist() == [0x7E] * 5 + [0xFE] * 2
