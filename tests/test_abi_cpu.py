"""The C ABI without a device: the library loads, exports every entry point
of include/sattn.h, sizes buffers, unpacks host copies and rejects invalid
arguments before any device call."""
import ctypes
import os
import re

import numpy as np
import pytest

import precision_flash_attention_amd as sattn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sattn.h")

OK, INVALID, UNSUPPORTED, SMALL, DEVICE = 0, 1, 2, 3, 4


@pytest.fixture(scope="module")
def lib():
    return sattn._load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sattn_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert sattn.abi_version() == 2
    for s in range(6):
        assert lib.sattn_status_string(s)
    assert lib.sattn_status_string(99) == b"unknown status"


def _sizes(B, H, Nq, Nkv):
    tile = 128 * 128
    nbq, nbk = -(-Nq // 128), -(-Nkv // 128)
    a = lambda x: (x + 255) // 256 * 256  # noqa: E731
    bh = B * H
    packed = (a(bh * nbq * tile) + a(bh * nbk * tile) * 2 + a(bh * nbq * 4) + a(bh * nbk * 4)
              + a(bh * 128 * 4) * 2)
    ws = a(bh * nbk * 128 * 4) * 2
    return packed, ws


@pytest.mark.parametrize("shape", [(1, 2, 256, 256), (1, 24, 4608, 4608), (2, 40, 32760, 512),
                                   (1, 40, 32760, 32760), (1, 24, 65520, 65520), (3, 1, 1, 1)])
def test_packed_bytes(shape):
    assert sattn.packed_bytes(*shape) == _sizes(*shape)


def test_packed_bytes_errors(lib):
    pb = ctypes.c_size_t()
    assert lib.sattn_packed_bytes(1, 1, 128, 128, 64, ctypes.byref(pb), None) == UNSUPPORTED
    assert lib.sattn_packed_bytes(0, 1, 128, 128, 128, ctypes.byref(pb), None) == INVALID
    assert lib.sattn_packed_bytes(1, -1, 128, 128, 128, ctypes.byref(pb), None) == INVALID
    assert lib.sattn_packed_bytes(1, 1, (1 << 24) + 1, 128, 128, ctypes.byref(pb), None) == UNSUPPORTED
    assert lib.sattn_packed_bytes(1 << 30, 1 << 30, 128, 128, 128, ctypes.byref(pb), None) == INVALID
    assert lib.sattn_packed_bytes(1, 1, 1, 1, 128, None, None) == OK
    # block-count limit 2^22: every launch's work-item count stays below 2^32
    assert lib.sattn_packed_bytes(1, 1 << 15, 1 << 14, 1 << 14, 128, None, None) == OK
    assert lib.sattn_packed_bytes(1, (1 << 15) + 1, 1 << 14, 128, 128, None, None) == UNSUPPORTED
    assert lib.sattn_packed_bytes(2, 1 << 15, 128, 1 << 14, 128, None, None) == UNSUPPORTED
    with pytest.raises(NotImplementedError):
        sattn.packed_bytes(1, 1, 128, 128, 64)
    with pytest.raises(ValueError):
        sattn.packed_bytes(1, 0, 128, 128)


ALIGNED = 1 << 20  # never dereferenced: validation must fail before any access


def quant_call(lib, **kw):
    a = dict(q=ALIGNED, k=ALIGNED, v=ALIGNED, B=1, H=2, Nq=256, Nkv=256, D=128, qs=None, ks=None,
             vs=None, packed=ALIGNED, pbytes=1 << 40, ws=ALIGNED, wbytes=1 << 40, stream=None)
    a.update(kw)
    return lib.sattn_quantize_qkv(a["q"], a["k"], a["v"], a["B"], a["H"], a["Nq"], a["Nkv"], a["D"],
                                  a["qs"], a["ks"], a["vs"], a["packed"], a["pbytes"], a["ws"],
                                  a["wbytes"], a["stream"])


def strides(*s):
    return (ctypes.c_int64 * 3)(*s)


def test_quantize_validation(lib):
    assert quant_call(lib, D=64) == UNSUPPORTED
    assert quant_call(lib, B=0) == INVALID
    assert quant_call(lib, q=None) == INVALID
    assert quant_call(lib, ws=None) == INVALID
    assert quant_call(lib, k=ALIGNED + 8) == INVALID
    assert quant_call(lib, packed=ALIGNED + 4) == INVALID
    assert quant_call(lib, pbytes=100) == SMALL
    assert quant_call(lib, wbytes=100) == SMALL
    assert quant_call(lib, qs=strides(65536, 256, 129)) == INVALID
    assert quant_call(lib, vs=strides(-8, 256, 128)) == INVALID
    assert quant_call(lib, Nkv=(1 << 24) + 1) == UNSUPPORTED
    # everything valid: the next step is the device check, which fails here
    assert quant_call(lib, qs=strides(65536, 256, 128)) == DEVICE


def fwd_call(lib, cross=False, **kw):
    a = dict(packed=ALIGNED, pbytes=1 << 40, B=1, H=2, Nq=256, Nkv=256, D=128, scale=0.088,
             out=ALIGNED, os=None, stream=None)
    a.update(kw)
    if cross:
        return lib.sattn_fwd_cross(a["packed"], a["pbytes"], a["B"], a["H"], a["Nq"], a["Nkv"], a["D"],
                                   ctypes.c_float(a["scale"]), a["out"], a["os"], a["stream"])
    return lib.sattn_fwd(a["packed"], a["pbytes"], a["B"], a["H"], a["Nq"], a["D"],
                         ctypes.c_float(a["scale"]), a["out"], a["os"], a["stream"])


@pytest.mark.parametrize("cross", [False, True])
def test_forward_validation(lib, cross):
    assert fwd_call(lib, cross, D=100) == UNSUPPORTED
    assert fwd_call(lib, cross, H=0) == INVALID
    assert fwd_call(lib, cross, packed=None) == INVALID
    assert fwd_call(lib, cross, out=None) == INVALID
    assert fwd_call(lib, cross, out=ALIGNED + 2) == INVALID
    assert fwd_call(lib, cross, scale=float("nan")) == INVALID
    assert fwd_call(lib, cross, scale=float("inf")) == INVALID
    assert fwd_call(lib, cross, scale=0.0) == INVALID
    assert fwd_call(lib, cross, scale=-1.0) == INVALID
    assert fwd_call(lib, cross, pbytes=1000) == SMALL
    assert fwd_call(lib, cross, os=strides(1 << 20, 100, 128)) == INVALID
    assert fwd_call(lib, cross) == DEVICE


def fwd_ex(lib, cross, **kw):
    a = dict(packed=ALIGNED, pbytes=1 << 40, fmt=0, B=1, H=2, Nq=256, Nkv=256, D=128, scale=0.088,
             out=ALIGNED, os=None, lse=None, splits=1, ws=None, wbytes=0, stream=None)
    a.update(kw)
    tail = (ctypes.c_float(a["scale"]), a["out"], a["os"], a["lse"], a["splits"], a["ws"], a["wbytes"],
            a["stream"])
    if cross:
        return lib.sattn_fwd_cross_ex(a["packed"], a["pbytes"], a["fmt"], a["B"], a["H"], a["Nq"], a["Nkv"],
                                      a["D"], *tail)
    return lib.sattn_fwd_ex(a["packed"], a["pbytes"], a["fmt"], a["B"], a["H"], a["Nq"], a["D"], *tail)


def _split_sizes(B, H, Nq, Nkv, num_splits):
    """Reference of the split rule as documented in include/sattn.h: the
    automatic choice splits only launches of fewer than 256 workgroups, into
    at most 256 // workgroups ranges of at least 8 tiles; every range holds a
    tile; the partials take 128 FP32 + 1 FP32 per (range, row)."""
    nbk = -(-Nkv // 128)
    want = num_splits
    if want == 0:
        g1 = B * H * -(-Nq // 256)
        want = max(1, min(256 // g1, nbk // 8)) if g1 < 256 else 1
    want = min(want, nbk)
    tps = -(-nbk // want)
    used = -(-nbk // tps)
    a = lambda x: (x + 255) // 256 * 256  # noqa: E731
    return (0 if used == 1 else a(used * B * H * Nq * 512) + a(used * B * H * Nq * 4)), used


@pytest.mark.parametrize("shape", [(1, 40, 256, 32760), (1, 40, 32760, 32760), (1, 2, 256, 256),
                                   (2, 3, 64, 4608), (1, 1, 1, 1 << 20), (1, 40, 256, 1000), (3, 5, 700, 9000)])
@pytest.mark.parametrize("num_splits", [0, 1, 2, 7, 256])
def test_split_workspace_sizes(shape, num_splits):
    assert sattn.fwd_workspace_bytes(*shape, num_splits=num_splits) == _split_sizes(*shape, num_splits)


def test_split_and_lse_validation(lib):
    wb = ctypes.c_size_t()
    assert lib.sattn_fwd_workspace_bytes(1, 2, 256, 256, 128, -1, ctypes.byref(wb), None) == INVALID
    assert lib.sattn_fwd_workspace_bytes(1, 2, 256, 256, 128, 257, ctypes.byref(wb), None) == INVALID
    assert lib.sattn_fwd_workspace_bytes(1, 2, 256, 256, 64, 1, ctypes.byref(wb), None) == UNSUPPORTED
    big, used = sattn.fwd_workspace_bytes(1, 2, 256, 8192, num_splits=4)
    assert used == 4 and big > 0
    for cross in (False, True):
        kw = dict(Nq=256, Nkv=8192) if cross else dict(Nq=8192, Nkv=8192)
        size, _ = sattn.fwd_workspace_bytes(1, 2, kw["Nq"], kw["Nkv"], num_splits=4)
        assert fwd_ex(lib, cross, splits=-1, **kw) == INVALID
        assert fwd_ex(lib, cross, splits=257, **kw) == INVALID
        assert fwd_ex(lib, cross, splits=4, **kw) == INVALID            # no workspace
        assert fwd_ex(lib, cross, splits=4, ws=ALIGNED + 8, wbytes=size, **kw) == INVALID
        assert fwd_ex(lib, cross, splits=4, ws=ALIGNED, wbytes=size - 1, **kw) == SMALL
        assert fwd_ex(lib, cross, splits=4, ws=ALIGNED, wbytes=size, **kw) == DEVICE
        assert fwd_ex(lib, cross, lse=ALIGNED + 2, **kw) == INVALID
        assert fwd_ex(lib, cross, lse=ALIGNED + 4, **kw) == DEVICE
        assert fwd_ex(lib, cross, splits=1, **kw) == DEVICE            # no split: no workspace needed


def _lut_bytes(B, H, Nq, Nkv):
    a = lambda x: (x + 255) // 256 * 256  # noqa: E731
    g = B * H * -(-Nq // 256)
    return a(4 * g) + a(4 * g * -(-Nkv // 128))


@pytest.mark.parametrize("shape", [(1, 2, 300, 700), (2, 40, 32760, 32760), (1, 1, 1, 1), (3, 5, 257, 129)])
def test_block_lut_sizes(shape):
    assert sattn.block_lut_bytes(*shape) == _lut_bytes(*shape)


def test_sparse_validation(lib):
    n = _lut_bytes(1, 2, 300, 700)
    assert lib.sattn_block_lut(None, 1, 2, 300, 700, 128, ALIGNED, n, None) == INVALID
    assert lib.sattn_block_lut(ALIGNED, 1, 2, 300, 700, 128, None, n, None) == INVALID
    assert lib.sattn_block_lut(ALIGNED, 1, 2, 300, 700, 128, ALIGNED + 4, n, None) == INVALID
    assert lib.sattn_block_lut(ALIGNED, 1, 2, 300, 700, 128, ALIGNED, n - 1, None) == SMALL
    assert lib.sattn_block_lut(ALIGNED, 1, 2, 300, 700, 64, ALIGNED, n, None) == UNSUPPORTED
    assert lib.sattn_block_lut(ALIGNED, 1, 2, 300, 700, 128, ALIGNED, n, None) == DEVICE

    def fs(**kw):
        a = dict(packed=ALIGNED, pbytes=1 << 40, fmt=0, D=128, scale=0.088, lut=ALIGNED, lbytes=n,
                 out=ALIGNED, lse=None)
        a.update(kw)
        return lib.sattn_fwd_sparse(a["packed"], a["pbytes"], a["fmt"], 1, 2, 300, 700, a["D"],
                                    ctypes.c_float(a["scale"]), a["lut"], a["lbytes"], a["out"], None,
                                    a["lse"], None)
    assert fs(lut=None) == INVALID
    assert fs(lut=ALIGNED + 8) == INVALID
    assert fs(lbytes=n - 1) == SMALL
    assert fs(fmt=3) == INVALID
    assert fs(D=64) == UNSUPPORTED
    assert fs(scale=0.0) == INVALID
    assert fs(lse=ALIGNED + 1) == INVALID
    assert fs(pbytes=10) == SMALL
    assert fs() == DEVICE


def test_format_entry_points_validation(lib):
    """The _ex calls take the Q/K code format (0 = INT8, 1 = FP8); any other
    value is an invalid argument, checked before the device."""
    q = dict(q=ALIGNED, k=ALIGNED, v=ALIGNED)
    st = strides(65536, 256, 128)
    for fmt, want in ((0, DEVICE), (1, DEVICE), (2, INVALID), (-1, INVALID)):
        assert lib.sattn_quantize_qkv_ex(q["q"], q["k"], q["v"], 1, 2, 256, 256, 128, st, None, None, fmt,
                                         ALIGNED, 1 << 40, ALIGNED, 1 << 40, None) == want, fmt
        assert fwd_ex(lib, False, fmt=fmt) == want, fmt
        assert fwd_ex(lib, True, fmt=fmt) == want, fmt
    # the shape checks come first, as in the calls without a format
    assert fwd_ex(lib, False, D=64) == UNSUPPORTED
    assert lib.sattn_quantize_qkv_ex(q["q"], q["k"], q["v"], 1, 2, 256, 256, 128, st, None, None, 1,
                                     ALIGNED, 100, ALIGNED, 1 << 40, None) == SMALL
    with pytest.raises(ValueError):
        sattn._format("int4")


def test_e4m3_validation(lib):
    assert lib.sattn_e4m3_encode(None, ALIGNED, 10, None) == INVALID
    assert lib.sattn_e4m3_encode(ALIGNED, ALIGNED, 0, None) == INVALID
    assert lib.sattn_e4m3_encode(ALIGNED, ALIGNED, 10, None) == DEVICE


def test_unpack_host_is_a_permutation_of_each_tile():
    B, H, Nq, Nkv = 1, 2, 256, 384
    pb, _ = sattn.packed_bytes(B, H, Nq, Nkv)
    rng = np.random.default_rng(0)
    host = rng.integers(0, 256, size=pb, dtype=np.uint8)
    # scale sections hold floats: write recognisable values
    lib = sattn._load()
    out = {
        "q8": np.empty((B, H, Nq, 128), np.int8), "k8": np.empty((B, H, Nkv, 128), np.int8),
        "v8": np.empty((B, H, Nkv, 128), np.uint8), "q_scale": np.empty((B, H, 2), np.float32),
        "k_scale": np.empty((B, H, 3), np.float32), "v_scale": np.empty((B, H, 128), np.float32),
        "k_mean": np.empty((B, H, 128), np.float32)}
    assert lib.sattn_unpack_host(host.ctypes.data, host.size, B, H, Nq, Nkv, 128,
                                 *(out[n].ctypes.data for n in ("q8", "k8", "v8", "q_scale", "k_scale",
                                                                "v_scale", "k_mean"))) == OK
    tile = 128 * 128
    # tiles are laid out q8 | k8 | v8, each [B][H][nb] tiles of 16 KiB
    off = 0
    for name, nb in (("q8", 2), ("k8", 3), ("v8", 3)):
        for bh in range(B * H):
            for t in range(nb):
                raw = host[off + (bh * nb + t) * tile: off + (bh * nb + t + 1) * tile]
                canon = out[name][0, bh, 128 * t: 128 * (t + 1)].view(np.uint8).ravel()
                assert np.array_equal(np.sort(raw), np.sort(canon)), (name, bh, t)
                if name == "v8":
                    # each V^T tile row (one channel) holds that channel's 128 keys
                    for d in (0, 5, 127):
                        assert np.array_equal(np.sort(raw[128 * d: 128 * d + 128]),
                                              np.sort(out["v8"][0, bh, 128 * t: 128 * t + 128, d]))
                else:
                    # each K/Q tile row (one token) holds that token's 128 channels
                    for r in (0, 9, 127):
                        assert np.array_equal(np.sort(raw[128 * r: 128 * r + 128]),
                                              np.sort(out[name][0, bh, 128 * t + r].view(np.uint8)))
        off += (B * H * nb * tile + 255) // 256 * 256
    assert lib.sattn_unpack_host(host.ctypes.data, 100, B, H, Nq, Nkv, 128, *([None] * 7)) == SMALL
    assert lib.sattn_unpack_host(None, host.size, B, H, Nq, Nkv, 128, *([None] * 7)) == INVALID


def test_python_layer_rejections():
    import torch
    q = torch.zeros(1, 8, 1, 128, dtype=torch.bfloat16)
    with pytest.raises(NotImplementedError):
        sattn.attention(q, q, q, causal=True)
    with pytest.raises(NotImplementedError):
        sattn.attention(q, q, q, attn_mask=torch.ones(1))
    with pytest.raises(NotImplementedError):
        sattn.attention(q, q, q, dropout_p=0.1)
    with pytest.raises(NotImplementedError):
        sattn.attention(q, q, q, cu_seqlens=torch.tensor([0, 8]))
    with pytest.raises(NotImplementedError):
        sattn.quantize_qkv(q.half(), q.half(), q.half())
    with pytest.raises(ValueError):
        sattn.quantize_qkv(q, q, q)  # host tensors
    with pytest.raises(ValueError):
        sattn.quantize_qkv(q.float(), q.float(), q.float())


def test_product_does_not_reference_the_oracle():
    pkg = os.path.join(ROOT, "precision_flash_attention_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), f
                assert "testkit" not in text, f


def test_q_smoothing_sizes_and_flags(lib):
    # the option adds the block means; then, with INT8 codes, four int8 digit
    # rows and 8 parameters per Q block, and with E4M3 codes the Delta-S table
    B, H, Nq, Nkv = 2, 3, 300, 700
    base = sattn.packed_bytes(B, H, Nq, Nkv)[0]
    nbq, nbk = 3, 6
    a = lambda x: (x + 255) // 256 * 256  # noqa: E731
    means = a(B * H * nbq * 128 * 4)
    assert (sattn.packed_bytes(B, H, Nq, Nkv, q_smooth=True)[0]
            == base + means + a(B * H * nbq * 512) + a(B * H * nbq * 8 * 4))
    assert (sattn.packed_bytes(B, H, Nq, Nkv, qk_format="fp8", q_smooth=True)[0]
            == base + means + a(B * H * nbq * nbk * 128 * 4))
    pb = ctypes.c_size_t()
    assert lib.sattn_packed_bytes_ex(1, 2, 256, 256, 128, 0x20, ctypes.byref(pb), None) == INVALID
    assert lib.sattn_packed_bytes_ex(1, 2, 256, 256, 128, 0x12, ctypes.byref(pb), None) == INVALID
    # a Delta-S table beyond 2^40 bytes is refused; the INT8 form has none
    assert lib.sattn_packed_bytes_ex(1, 1, 1 << 24, 1 << 24, 128, 0x11, ctypes.byref(pb), None) == UNSUPPORTED
    assert lib.sattn_packed_bytes_ex(1, 1, 1 << 24, 1 << 24, 128, 0x10, ctypes.byref(pb), None) == OK
    st = strides(65536, 256, 128)
    small = sattn.packed_bytes(1, 2, 256, 256)[0]   # enough without smoothing only
    assert lib.sattn_quantize_qkv_ex(ALIGNED, ALIGNED, ALIGNED, 1, 2, 256, 256, 128, st, None, None, 0x10,
                                     ALIGNED, small, ALIGNED, 1 << 40, None) == SMALL
    assert lib.sattn_quantize_qkv_ex(ALIGNED, ALIGNED, ALIGNED, 1, 2, 256, 256, 128, st, None, None, 0x11,
                                     ALIGNED, 1 << 40, ALIGNED, 1 << 40, None) == DEVICE
    assert fwd_ex(lib, False, fmt=0x10, pbytes=sattn.packed_bytes(1, 2, 256, 256)[0]) == SMALL
    assert fwd_ex(lib, False, fmt=0x11) == DEVICE
    n = _lut_bytes(1, 2, 256, 256)
    assert lib.sattn_fwd_sparse(ALIGNED, 1 << 40, 0x10, 1, 2, 256, 256, 128, ctypes.c_float(0.088), ALIGNED, n,
                                ALIGNED, None, None, None) == UNSUPPORTED
    assert lib.sattn_unpack_q_mean_host(None, 10, 1, 2, 256, 256, 128, ALIGNED) == INVALID
    assert lib.sattn_unpack_q_mean_host(ALIGNED, 10, 1, 2, 256, 256, 128, ALIGNED) == SMALL
