"""GPU preprocessing parity: INT8/E4M3 codes, FP32 scales and the K mean are
bit-exact against the oracle for every workload at its full size, for ragged
tails, strided layouts and adversarial blocks."""
import numpy as np
import pytest

import oracle
import precision_flash_attention_amd as sattn
import testkit
from gpu_helpers import assert_codes_equal, log, to_dev, workload

pytestmark = pytest.mark.gpu


def gpu_codes(q, k, v, qk_format="int8"):
    p = sattn.quantize_qkv(to_dev(q), to_dev(k), to_dev(v), qk_format=qk_format)
    return sattn.unpack_host(p)


@pytest.mark.parametrize("cfg_index", [1, 2, 3, 4, 5])
def test_codes_bit_exact_full_size(device, cfg_index):
    log(f"quantize parity, workload {cfg_index}")
    cfg, q, k, v, want = workload(cfg_index)
    assert_codes_equal(gpu_codes(q, k, v), want)


@pytest.mark.parametrize("N", [1, 2, 127, 128, 129, 255, 257, 1000])
def test_codes_ragged_tails(device, N):
    log(f"quantize tails N={N}")
    cfg = testkit.CONFIGS[4]
    q, k, v = testkit.make_inputs(cfg, seed=100 + N, H=3, Nq=N, Nkv=N)
    assert_codes_equal(gpu_codes(q, k, v), oracle.quantize(q, k, v))


@pytest.mark.parametrize("Nq,Nkv", [(300, 512), (1, 129), (129, 1), (640, 77)])
def test_codes_cross_shapes(device, Nq, Nkv):
    log(f"quantize cross Nq={Nq} Nkv={Nkv}")
    cfg = testkit.CONFIGS[3]
    q, k, v = testkit.make_inputs(cfg, seed=7, B=2, H=2, Nq=Nq, Nkv=Nkv)
    assert_codes_equal(gpu_codes(q, k, v), oracle.quantize(q, k, v))


def test_strided_inputs_give_the_same_codes(device):
    import torch
    log("quantize strided layouts")
    cfg = testkit.CONFIGS[2]
    q, k, v = testkit.make_inputs(cfg, H=4, Nq=300, Nkv=300)
    want = oracle.quantize(q, k, v)
    # BHSD storage viewed as BSHD, and a head slice of a wider tensor
    qd, kd, vd = (to_dev(t) for t in (q, k, v))
    qb = qd.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    wide = torch.zeros(1, 300, 9, 128, dtype=torch.bfloat16, device="cuda:0")
    wide[:, :, 3:7] = kd
    kh = wide[:, :, 3:7]
    assert not qb.is_contiguous() and not kh.is_contiguous()
    p = sattn.quantize_qkv(qb, kh, vd)
    assert_codes_equal(sattn.unpack_host(p), want)
    # 3D input (B = 1)
    p3 = sattn.quantize_qkv(qd[0], kd[0], vd[0])
    assert_codes_equal(sattn.unpack_host(p3), want)


def _bf16(x):
    f = np.asarray(x, np.float32)
    u = f.view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("qk_format", ["int8", "fp8"])
def test_adversarial_blocks(device, qk_format):
    log(f"quantize adversarial blocks ({qk_format} Q/K)")
    rng = np.random.default_rng(5)
    N, H = 512, 4
    q = np.zeros((1, N, H, 128), np.float32)
    k = np.zeros_like(q)
    v = np.zeros_like(q)
    # head 0: block 0 exact half-integer quotients (scale 1: amax 127)
    q[0, :128, 0] = rng.integers(-254, 255, size=(128, 128)) / 2.0
    q[0, 0, 0, 0] = 127.0
    # block 1 all zero; block 2 subnormal BF16 values; block 3 huge range
    q[0, 256:384, 0] = rng.integers(-100, 100, size=(128, 128)) * 2.0 ** -133
    q[0, 384:, 0] = rng.normal(size=(128, 128)) * 10.0 ** rng.uniform(-30, 30, size=(128, 128))
    # V channels whose quotients land on E4M3 midpoints: amax 448 -> scale 1
    mids = []
    for e in range(-6, 8):
        for m in range(8):
            mids.append((1 + (2 * m + 1) / 16) * 2.0 ** e)
    mids = np.array(mids)
    v[0, :, 0] = rng.choice(np.concatenate([mids, -mids, [448.0]]), size=(N, 128))
    v[0, 0, 0, :] = 448.0
    v[0, :, 1] = rng.normal(size=(N, 128)) * 1e-3   # tiny channel scales
    v[0, :, 2, :64] = 0.0                           # zero channels
    v[0, :, 2, 64:] = -0.0
    v[0, :, 3] = rng.normal(size=(N, 128)) * 2.0 ** -128
    # K: bias much larger than the spread (smoothing cancels it)
    k[0, :, :] = 300.0 + rng.normal(size=(N, H, 128))
    k[0, :, 1] = rng.normal(size=(N, 128)) * 2.0 ** -125
    q[0, :, 1:] = rng.normal(size=(N, H - 1, 128))
    qb, kb, vb = _bf16(q), _bf16(k), _bf16(v)
    assert_codes_equal(gpu_codes(qb, kb, vb, qk_format), oracle.quantize(qb, kb, vb, qk_format=qk_format))


def test_deterministic(device):
    log("quantize determinism")
    cfg = testkit.CONFIGS[4]
    q, k, v = testkit.make_inputs(cfg, H=8, Nq=4096, Nkv=4096)
    a = sattn.quantize_qkv(to_dev(q), to_dev(k), to_dev(v))
    b = sattn.quantize_qkv(to_dev(q), to_dev(k), to_dev(v))
    import torch
    torch.cuda.synchronize()
    assert torch.equal(a.buf, b.buf)
