"""The allocation-free quantize entry point against the one with a caller
workspace: sattn_quantize_qkv_noalloc (static device workspace) must give
the packed buffer of sattn_quantize_qkv_ex bit for bit.  Two calls in a row
(the static workspace keeps the first call's contents), the second smaller
and in the other Q/K format; then a problem whose workspace exceeds the
static array is refused before any device work."""
import ctypes

import numpy as np
import pytest
import torch

import precision_flash_attention_amd as sattn
import testkit
from gpu_helpers import log, to_dev

pytestmark = pytest.mark.gpu


def _both(q, k, v, fmt):
    # both packed buffers start from the same non-zero fill, so that the
    # alignment gaps between sections (never written) compare equal and
    # every byte the quantizer writes is checked
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    B, Nq, H, _ = q.shape
    pb, _ = sattn.packed_bytes(B, H, Nq, k.shape[1], qk_format=fmt)
    ref = sattn.quantize_qkv(qd, kd, vd, packed=torch.full((pb,), 0xA5, dtype=torch.uint8, device="cuda:0"),
                             qk_format=fmt)
    got = sattn.quantize_qkv_noalloc(qd, kd, vd, torch.full((pb,), 0xA5, dtype=torch.uint8, device="cuda:0"),
                                     qk_format=fmt)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("first,second", [((2, 3, 700, 1300, "int8"), (1, 2, 200, 333, "fp8"))])
def test_noalloc_equals_caller_workspace(device, first, second):
    for i, (B, H, Nq, Nkv, fmt) in enumerate((first, second)):
        q, k, v = testkit.make_inputs(testkit.CONFIGS[4], seed=600 + i, B=B, H=H, Nq=Nq, Nkv=Nkv)
        ref, got = _both(q, k, v, fmt)
        same = torch.equal(ref.buf, got.buf)
        log(f"  call {i + 1}: B={B} H={H} Nq={Nq} Nkv={Nkv} [{fmt}]: packed buffers equal: {same}")
        assert same
        # and the attention results from both buffers
        a = sattn.fwd_cross(ref, 1.0 / np.sqrt(128.0))
        b = sattn.fwd_cross(got, 1.0 / np.sqrt(128.0))
        assert torch.equal(a, b)


def test_noalloc_refuses_beyond_the_static_workspace(device):
    lib = sattn._load()
    # B*H*ceil(Nkv/128) = 16385 blocks need 16385 * 1 KiB > 16 MiB of workspace
    B, H, N = 1, 16385, 128
    _, wb = sattn.packed_bytes(B, H, N, N)
    assert wb > (16 << 20)
    aligned = 1 << 20                                  # never dereferenced
    st = lib.sattn_quantize_qkv_noalloc(aligned, aligned, aligned, B, H, N, N, 128, None, None, None, 0,
                                        aligned, 1 << 62, None)
    assert st == 2  # SATTN_ERR_UNSUPPORTED
