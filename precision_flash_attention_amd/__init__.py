"""INT8-QK / FP8-PV ("SageAttention-style") attention forward for MI355X.

A thin binding over the C ABI of ``libsattn.so`` (``include/sattn.h``): it
only marshals arguments.  PyTorch supplies device memory and the current
stream; every step of the computation runs in the library's HIP kernels, and
there is no other code path -- if the library is missing or the device is not
gfx950, calls raise.

Entry points (same names as the C ABI):
    quantize_qkv(q, k, v, qk_format)     -> Packed   (preprocessing)
    fwd(packed, softmax_scale, out)      -> Tensor   (self-attention)
    fwd_cross(packed, softmax_scale, out)-> Tensor   (cross-attention)
    attention(q, k, v, softmax_scale, out, qk_format=...)  (both stages)
    fwd_workspace_bytes(B, H, Nq, Nkv, num_splits) -> (bytes, splits)
    block_lut(block_mask, Nq, Nkv)       -> BlockLut (block-sparse table)
    fwd_sparse(packed, lut, softmax_scale, out)  (block-sparse attention)

The forward calls take ``return_lse`` (also return the FP32 [B, H, Nq]
log-sum-exp of each row's logits, the FA4 autotuning page's float32 LSE) and
``num_splits`` (split-KV: 1 = none, the default; 0 = the library's choice;
k = at most k key ranges; the binding allocates the partials' workspace
unless one is passed).

``qk_format`` is "int8" (INT8 Q/K codes, scale amax/127: the gfx1201 backend
page's INT8/FP8/BF16 path) or "fp8" (E4M3 Q/K codes, scale amax/448: the
FP8/FP8/BF16 row of the MHA v4 page's MI355X table); ``q_smooth=True`` adds
Q smoothing per 128-token block with the Delta-S correction.  A Packed buffer records
its format and the forward calls pass it on (the ``_ex`` C entry points).

As the gfx1201 backend page specifies its backend ("[ROCm] Add
aiter_sage_attn attention backend for gfx1201 (RDNA4)", Changes): BF16
Q/K/V, head dim 128, non-causal, ``softmax_scale`` passed through; causal,
masks, dropout and packed multi-sequence ``cu_seqlens`` raise instead of
computing something else.  FP16 inputs are not supported by this library.
Optional arguments use ``Optional[...]`` annotations (the MHA v4 page's lint
comments and the AITER bump page both concern PEP 604 unions breaking
Dynamo).  3D ``[N, H, D]`` and 4D ``[B, N, H, D]`` inputs are accepted.
"""
import ctypes
import math
import os
from dataclasses import dataclass
from typing import Dict, Optional, Tuple

import torch

__all__ = ["Packed", "SattnError", "QK_FORMATS", "abi_version", "packed_bytes", "quantize_qkv",
           "quantize_qkv_noalloc", "fwd",
           "fwd_cross", "attention", "fwd_workspace_bytes", "BlockLut", "block_lut_bytes", "block_lut",
           "fwd_sparse", "unpack_host", "e4m3_encode", "library_path"]

HERE = os.path.dirname(os.path.abspath(__file__))
# SATTN_LIBRARY: load another build of the library (the host-sanitizer test's)
_LIB_PATH = os.environ.get("SATTN_LIBRARY") or os.path.join(HERE, "libsattn.so")
_lib = None

SATTN_OK = 0
SATTN_ERR_INVALID_ARGUMENT = 1
SATTN_ERR_UNSUPPORTED = 2
SATTN_ERR_BUFFER_TOO_SMALL = 3
SATTN_ERR_DEVICE = 4
SATTN_ERR_LAUNCH = 5
HEAD_DIM = 128
QK_FORMATS = {"int8": 0, "fp8": 1}  # sattn_qk_format
QK_SMOOTH_Q = 0x10                  # SATTN_QK_SMOOTH_Q

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I64P = ctypes.POINTER(ctypes.c_int64)
_SZ = ctypes.c_size_t


class SattnError(RuntimeError):
    """A device-side failure reported by libsattn (no device, launch error)."""


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"libsattn.so is not built ({_LIB_PATH}); run "
                               "`python precision_flash_attention_amd/build.py` first")
        lib = ctypes.CDLL(_LIB_PATH)
        lib.sattn_abi_version.restype = ctypes.c_int
        lib.sattn_status_string.argtypes = [ctypes.c_int]
        lib.sattn_status_string.restype = ctypes.c_char_p
        lib.sattn_packed_bytes.argtypes = [_I64] * 5 + [ctypes.POINTER(_SZ)] * 2
        lib.sattn_packed_bytes_ex.argtypes = [_I64] * 5 + [ctypes.c_int] + [ctypes.POINTER(_SZ)] * 2
        lib.sattn_unpack_q_mean_host.argtypes = [_P, _SZ] + [_I64] * 5 + [_P]
        lib.sattn_quantize_qkv.argtypes = [_P, _P, _P] + [_I64] * 5 + [_I64P] * 3 + [_P, _SZ, _P, _SZ, _P]
        lib.sattn_fwd.argtypes = [_P, _SZ] + [_I64] * 4 + [ctypes.c_float, _P, _I64P, _P]
        lib.sattn_fwd_cross.argtypes = [_P, _SZ] + [_I64] * 5 + [ctypes.c_float, _P, _I64P, _P]
        lib.sattn_quantize_qkv_noalloc.argtypes = ([_P, _P, _P] + [_I64] * 5 + [_I64P] * 3 + [ctypes.c_int]
                                                   + [_P, _SZ, _P])
        lib.sattn_quantize_qkv_ex.argtypes = ([_P, _P, _P] + [_I64] * 5 + [_I64P] * 3 + [ctypes.c_int]
                                              + [_P, _SZ, _P, _SZ, _P])
        lib.sattn_fwd_ex.argtypes = ([_P, _SZ, ctypes.c_int] + [_I64] * 4
                                     + [ctypes.c_float, _P, _I64P, _P, ctypes.c_int, _P, _SZ, _P])
        lib.sattn_fwd_cross_ex.argtypes = ([_P, _SZ, ctypes.c_int] + [_I64] * 5
                                           + [ctypes.c_float, _P, _I64P, _P, ctypes.c_int, _P, _SZ, _P])
        lib.sattn_fwd_workspace_bytes.argtypes = ([_I64] * 5 + [ctypes.c_int, ctypes.POINTER(_SZ),
                                                                ctypes.POINTER(ctypes.c_int)])
        lib.sattn_block_lut_bytes.argtypes = [_I64] * 5 + [ctypes.POINTER(_SZ)]
        lib.sattn_block_lut.argtypes = [_P] + [_I64] * 5 + [_P, _SZ, _P]
        lib.sattn_fwd_sparse.argtypes = ([_P, _SZ, ctypes.c_int] + [_I64] * 5
                                         + [ctypes.c_float, _P, _SZ, _P, _I64P, _P, _P])
        lib.sattn_unpack_host.argtypes = [_P, _SZ] + [_I64] * 5 + [_P] * 7
        lib.sattn_e4m3_encode.argtypes = [_P, _P, _I64, _P]
        for f in ("sattn_packed_bytes", "sattn_packed_bytes_ex", "sattn_unpack_q_mean_host",
                  "sattn_quantize_qkv", "sattn_fwd", "sattn_fwd_cross",
                  "sattn_quantize_qkv_ex", "sattn_fwd_ex", "sattn_fwd_cross_ex", "sattn_fwd_workspace_bytes",
                  "sattn_block_lut_bytes", "sattn_block_lut", "sattn_fwd_sparse",
                  "sattn_unpack_host", "sattn_e4m3_encode"):
            getattr(lib, f).restype = ctypes.c_int
        _lib = lib
    return _lib


def _check(status: int, what: str) -> None:
    if status == SATTN_OK:
        return
    msg = f"{what}: {_load().sattn_status_string(status).decode()} (status {status})"
    if status in (SATTN_ERR_INVALID_ARGUMENT, SATTN_ERR_BUFFER_TOO_SMALL):
        raise ValueError(msg)
    if status == SATTN_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    raise SattnError(msg)


def abi_version() -> int:
    return int(_load().sattn_abi_version())


def packed_bytes(B: int, H: int, Nq: int, Nkv: int, D: int = HEAD_DIM, qk_format: str = "int8",
                 q_smooth: bool = False) -> Tuple[int, int]:
    """(packed bytes, workspace bytes) for a problem (Q smoothing adds the
    block means and the Delta-S table)."""
    pb, wb = _SZ(0), _SZ(0)
    _check(_load().sattn_packed_bytes_ex(B, H, Nq, Nkv, D, _format(qk_format, q_smooth), ctypes.byref(pb),
                                         ctypes.byref(wb)), "sattn_packed_bytes")
    return int(pb.value), int(wb.value)


@dataclass
class Packed:
    """Output of quantize_qkv: a device buffer in the library's packed layout."""
    buf: torch.Tensor
    B: int
    H: int
    Nq: int
    Nkv: int
    squeeze_batch: bool = False
    qk_format: str = "int8"
    q_smooth: bool = False


def _stream_ptr(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _as4d(x: torch.Tensor, name: str) -> Tuple[torch.Tensor, bool]:
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if x.dtype == torch.float16:
        raise NotImplementedError(f"{name}: FP16 inputs are not supported (BF16 only)")
    if x.dtype != torch.bfloat16:
        raise ValueError(f"{name} must be bfloat16, got {x.dtype}")
    if x.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if x.dim() == 3:
        return x.unsqueeze(0), True
    if x.dim() != 4:
        raise ValueError(f"{name} must be [B, N, H, D] or [N, H, D]")
    return x, False


def _strides(x: torch.Tensor):
    if x.stride(3) != 1:
        raise ValueError("the head dimension must be contiguous")
    return (ctypes.c_int64 * 3)(x.stride(0), x.stride(1), x.stride(2))


def _format(qk_format: str, q_smooth: bool = False) -> int:
    if qk_format not in QK_FORMATS:
        raise ValueError(f"qk_format must be one of {sorted(QK_FORMATS)}, got {qk_format!r}")
    return QK_FORMATS[qk_format] | (QK_SMOOTH_Q if q_smooth else 0)


def quantize_qkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                 packed: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None, qk_format: str = "int8",
                 q_smooth: bool = False) -> Packed:
    """BF16 q [B,Nq,H,128], k/v [B,Nkv,H,128] -> packed Q/K codes (INT8 or
    E4M3, per ``qk_format``), E4M3 V codes and scales."""
    fmt = _format(qk_format, q_smooth)
    q4, sq = _as4d(q, "q")
    k4, _ = _as4d(k, "k")
    v4, _ = _as4d(v, "v")
    B, Nq, H, D = q4.shape
    Nkv = k4.shape[1]
    if tuple(k4.shape) != (B, Nkv, H, D) or tuple(v4.shape) != (B, Nkv, H, D):
        raise ValueError(f"shape mismatch: q {tuple(q4.shape)} k {tuple(k4.shape)} v {tuple(v4.shape)}")
    if not (q4.device == k4.device == v4.device):
        raise ValueError("q, k, v must be on one device")
    pb, wb = packed_bytes(B, H, Nq, Nkv, D, qk_format, q_smooth)
    if packed is None:
        packed = torch.empty(pb, dtype=torch.uint8, device=q4.device)
    if workspace is None:
        workspace = torch.empty(wb, dtype=torch.uint8, device=q4.device)
    qs, ks, vs = _strides(q4), _strides(k4), _strides(v4)
    _check(_load().sattn_quantize_qkv_ex(q4.data_ptr(), k4.data_ptr(), v4.data_ptr(), B, H, Nq, Nkv, D,
                                         qs, ks, vs, fmt, packed.data_ptr(),
                                         packed.numel() * packed.element_size(), workspace.data_ptr(),
                                         workspace.numel() * workspace.element_size(),
                                         _stream_ptr(q4.device)), "sattn_quantize_qkv")
    return Packed(packed, B, H, Nq, Nkv, sq, qk_format, q_smooth)


def quantize_qkv_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, packed: torch.Tensor,
                         qk_format: str = "int8", q_smooth: bool = False) -> Packed:
    """As quantize_qkv into the caller's `packed` (uint8, packed_bytes long),
    with the library's static device workspace instead of a caller's
    (sattn_quantize_qkv_noalloc): nothing is allocated.  Calls that overlap
    on one GPU share that workspace and race."""
    fmt = _format(qk_format, q_smooth)
    q4, sq = _as4d(q, "q")
    k4, _ = _as4d(k, "k")
    v4, _ = _as4d(v, "v")
    B, Nq, H, D = q4.shape
    Nkv = k4.shape[1]
    if tuple(k4.shape) != (B, Nkv, H, D) or tuple(v4.shape) != (B, Nkv, H, D):
        raise ValueError(f"shape mismatch: q {tuple(q4.shape)} k {tuple(k4.shape)} v {tuple(v4.shape)}")
    qs, ks, vs = _strides(q4), _strides(k4), _strides(v4)
    _check(_load().sattn_quantize_qkv_noalloc(q4.data_ptr(), k4.data_ptr(), v4.data_ptr(), B, H, Nq, Nkv, D,
                                              qs, ks, vs, fmt, packed.data_ptr(),
                                              packed.numel() * packed.element_size(), _stream_ptr(q4.device)),
           "sattn_quantize_qkv_noalloc")
    return Packed(packed, B, H, Nq, Nkv, sq, qk_format, q_smooth)


def _scale(softmax_scale: Optional[float]) -> float:
    return 1.0 / math.sqrt(HEAD_DIM) if softmax_scale is None else float(softmax_scale)


def _out(p: Packed, out: Optional[torch.Tensor]) -> Tuple[torch.Tensor, torch.Tensor]:
    if out is None:
        o4 = torch.empty((p.B, p.Nq, p.H, HEAD_DIM), dtype=torch.bfloat16, device=p.buf.device)
        return (o4[0] if p.squeeze_batch else o4), o4
    o4, _ = _as4d(out, "out")
    if tuple(o4.shape) != (p.B, p.Nq, p.H, HEAD_DIM):
        raise ValueError(f"out has shape {tuple(o4.shape)}, expected {(p.B, p.Nq, p.H, HEAD_DIM)}")
    return out, o4


def fwd_workspace_bytes(B: int, H: int, Nq: int, Nkv: int, num_splits: int = 0) -> Tuple[int, int]:
    """(split-KV workspace bytes, key ranges used) of a forward call."""
    wb, used = _SZ(0), ctypes.c_int(0)
    _check(_load().sattn_fwd_workspace_bytes(B, H, Nq, Nkv, HEAD_DIM, int(num_splits), ctypes.byref(wb),
                                             ctypes.byref(used)), "sattn_fwd_workspace_bytes")
    return int(wb.value), int(used.value)


def _forward(name: str, packed: Packed, softmax_scale, out, return_lse: bool, num_splits: int,
             workspace: Optional[torch.Tensor]):
    res, o4 = _out(packed, out)
    dev = o4.device
    lse = torch.empty((packed.B, packed.H, packed.Nq), dtype=torch.float32, device=dev) if return_lse else None
    wb, _ = fwd_workspace_bytes(packed.B, packed.H, packed.Nq, packed.Nkv, num_splits)
    if workspace is None and wb > 0:
        workspace = torch.empty(wb, dtype=torch.uint8, device=dev)
    wptr = workspace.data_ptr() if workspace is not None else None
    wlen = workspace.numel() * workspace.element_size() if workspace is not None else 0
    common = (_scale(softmax_scale), o4.data_ptr(), _strides(o4), None if lse is None else lse.data_ptr(),
              int(num_splits), wptr, wlen, _stream_ptr(dev))
    lib = _load()
    if name == "sattn_fwd":
        st = lib.sattn_fwd_ex(packed.buf.data_ptr(), packed.buf.numel(), _format(packed.qk_format, packed.q_smooth),
                              packed.B, packed.H, packed.Nq, HEAD_DIM, *common)
    else:
        st = lib.sattn_fwd_cross_ex(packed.buf.data_ptr(), packed.buf.numel(), _format(packed.qk_format, packed.q_smooth),
                                    packed.B, packed.H, packed.Nq, packed.Nkv, HEAD_DIM, *common)
    _check(st, name)
    if not return_lse:
        return res
    return res, (lse[0] if packed.squeeze_batch else lse)


def fwd(packed: Packed, softmax_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
        return_lse: bool = False, num_splits: int = 1, workspace: Optional[torch.Tensor] = None):
    """Self-attention (Nq == Nkv) from a packed buffer; BF16 output (and the
    FP32 LSE [B, H, Nq] with return_lse)."""
    if packed.Nq != packed.Nkv:
        raise NotImplementedError("fwd needs Nq == Nkv; use fwd_cross")
    return _forward("sattn_fwd", packed, softmax_scale, out, return_lse, num_splits, workspace)


def fwd_cross(packed: Packed, softmax_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
              return_lse: bool = False, num_splits: int = 1, workspace: Optional[torch.Tensor] = None):
    """Cross-attention (any Nq, Nkv) from a packed buffer; BF16 output (and
    the FP32 LSE [B, H, Nq] with return_lse)."""
    return _forward("sattn_fwd_cross", packed, softmax_scale, out, return_lse, num_splits, workspace)


@dataclass
class BlockLut:
    """Output of block_lut: a device table in the library's layout."""
    buf: torch.Tensor
    B: int
    H: int
    Nq: int
    Nkv: int


def block_lut_bytes(B: int, H: int, Nq: int, Nkv: int) -> int:
    n = _SZ(0)
    _check(_load().sattn_block_lut_bytes(B, H, Nq, Nkv, HEAD_DIM, ctypes.byref(n)), "sattn_block_lut_bytes")
    return int(n.value)


def block_lut(block_mask: torch.Tensor, Nq: int, Nkv: int, out: Optional[torch.Tensor] = None) -> BlockLut:
    """Block mask [B, H, ceil(Nq/128), ceil(Nkv/128)] (bool or uint8, device;
    nonzero = attend) -> the table fwd_sparse reads."""
    if not isinstance(block_mask, torch.Tensor) or block_mask.device.type != "cuda":
        raise ValueError("block_mask must be a device tensor")
    if block_mask.dim() != 4:
        raise ValueError("block_mask must be [B, H, ceil(Nq/128), ceil(Nkv/128)]")
    B, H, nbq, nbk = block_mask.shape
    if (nbq, nbk) != ((Nq + 127) // 128, (Nkv + 127) // 128):
        raise ValueError(f"block_mask has {nbq} x {nbk} blocks, expected "
                         f"{(Nq + 127) // 128} x {(Nkv + 127) // 128}")
    m = block_mask.to(torch.uint8).contiguous()
    n = block_lut_bytes(B, H, Nq, Nkv)
    if out is None:
        out = torch.empty(n, dtype=torch.uint8, device=m.device)
    _check(_load().sattn_block_lut(m.data_ptr(), B, H, Nq, Nkv, HEAD_DIM, out.data_ptr(),
                                   out.numel() * out.element_size(), _stream_ptr(m.device)), "sattn_block_lut")
    return BlockLut(out, B, H, Nq, Nkv)


def fwd_sparse(packed: Packed, lut: BlockLut, softmax_scale: Optional[float] = None,
               out: Optional[torch.Tensor] = None, return_lse: bool = False):
    """Block-sparse attention over the blocks the table lists; BF16 output
    (and the FP32 LSE [B, H, Nq], -inf on rows without keys, with return_lse)."""
    if (lut.B, lut.H, lut.Nq, lut.Nkv) != (packed.B, packed.H, packed.Nq, packed.Nkv):
        raise ValueError("the block table was made for another problem shape")
    res, o4 = _out(packed, out)
    dev = o4.device
    lse = torch.empty((packed.B, packed.H, packed.Nq), dtype=torch.float32, device=dev) if return_lse else None
    _check(_load().sattn_fwd_sparse(packed.buf.data_ptr(), packed.buf.numel(), _format(packed.qk_format, packed.q_smooth),
                                    packed.B, packed.H, packed.Nq, packed.Nkv, HEAD_DIM, _scale(softmax_scale),
                                    lut.buf.data_ptr(), lut.buf.numel(), o4.data_ptr(), _strides(o4),
                                    None if lse is None else lse.data_ptr(), _stream_ptr(dev)), "sattn_fwd_sparse")
    if not return_lse:
        return res
    return res, (lse[0] if packed.squeeze_batch else lse)


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
              softmax_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
              causal: bool = False, attn_mask: Optional[torch.Tensor] = None,
              dropout_p: float = 0.0, cu_seqlens: Optional[torch.Tensor] = None,
              qk_format: str = "int8", return_lse: bool = False, num_splits: int = 1,
              q_smooth: bool = False):
    """Quantize and attend.  Rejects what this path does not compute."""
    if causal:
        raise NotImplementedError("causal attention is not supported")
    if attn_mask is not None:
        raise NotImplementedError("attention masks are not supported")
    if dropout_p != 0.0:
        raise NotImplementedError("dropout is not supported")
    if cu_seqlens is not None:
        raise NotImplementedError("packed multi-sequence (cu_seqlens) inputs are not supported")
    p = quantize_qkv(q, k, v, qk_format=qk_format, q_smooth=q_smooth)
    if p.Nq == p.Nkv:
        return fwd(p, softmax_scale, out, return_lse=return_lse, num_splits=num_splits)
    return fwd_cross(p, softmax_scale, out, return_lse=return_lse, num_splits=num_splits)


def unpack_host(packed: Packed) -> Dict[str, "object"]:
    """Copy a packed buffer to the host and return its canonical numpy arrays."""
    import numpy as np
    host = packed.buf.detach().cpu().numpy()
    B, H, Nq, Nkv = packed.B, packed.H, packed.Nq, packed.Nkv
    nbq, nbk = (Nq + 127) // 128, (Nkv + 127) // 128
    r = {
        "q8": np.empty((B, H, Nq, HEAD_DIM), np.int8),
        "k8": np.empty((B, H, Nkv, HEAD_DIM), np.int8),
        "v8": np.empty((B, H, Nkv, HEAD_DIM), np.uint8),
        "q_scale": np.empty((B, H, nbq), np.float32),
        "k_scale": np.empty((B, H, nbk), np.float32),
        "v_scale": np.empty((B, H, HEAD_DIM), np.float32),
        "k_mean": np.empty((B, H, HEAD_DIM), np.float32),
    }
    _check(_load().sattn_unpack_host(host.ctypes.data, host.size, B, H, Nq, Nkv, HEAD_DIM,
                                     *(r[n].ctypes.data for n in ("q8", "k8", "v8", "q_scale",
                                                                  "k_scale", "v_scale", "k_mean"))),
           "sattn_unpack_host")
    r["qk_format"] = packed.qk_format
    if packed.q_smooth:
        r["q_mean"] = np.empty((B, H, nbq, HEAD_DIM), np.float32)
        _check(_load().sattn_unpack_q_mean_host(host.ctypes.data, host.size, B, H, Nq, Nkv, HEAD_DIM,
                                                r["q_mean"].ctypes.data), "sattn_unpack_q_mean_host")
    return r


def e4m3_encode(x: torch.Tensor) -> torch.Tensor:
    """The device FP32 -> E4M3 conversion of the V quantizer (clamped to +-448)."""
    if x.dtype != torch.float32 or x.device.type != "cuda" or not x.is_contiguous():
        raise ValueError("x must be a contiguous float32 device tensor")
    out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _check(_load().sattn_e4m3_encode(x.data_ptr(), out.data_ptr(), x.numel(), _stream_ptr(x.device)),
           "sattn_e4m3_encode")
    return out
