"""CPU oracle for the INT8-QK / FP8-PV attention forward -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package; the product library never does.  The arithmetic lives in
sattn_oracle.c (plain C, FP64 where the method leaves precision open); this
file only marshals numpy arrays.

Canonical layouts: BF16 inputs BSHD uint16 [B, N, H, 128]; codes
[B, H, N, 128]; q/k scales [B, H, ceil(N/128)]; v scale and k mean [B, H, 128].
"""
import ctypes
import os
from typing import Dict, Optional, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# SATTN_ORACLE_LIB: another build of sattn_oracle.c (the sanitizer test's)
_LIB_PATH = os.environ.get("SATTN_ORACLE_LIB") or os.path.join(HERE, "liboracle.so")
_lib = None
D = 128
BLK = 128
P = ctypes.c_void_p
I64 = ctypes.c_int64


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.orc_e4m3_decode.restype = ctypes.c_double
        lib.orc_e4m3_encode.argtypes = [ctypes.c_float]
        lib.orc_e4m3_encode.restype = ctypes.c_uint8
        lib.orc_e4m3_encode_nearest.argtypes = [ctypes.c_float]
        lib.orc_e4m3_encode_nearest.restype = ctypes.c_uint8
        lib.orc_e4m3_sweep_mismatches.argtypes = [ctypes.c_uint32, ctypes.c_uint32]
        lib.orc_e4m3_sweep_mismatches.restype = ctypes.c_int64
        lib.orc_e4m3_encode_array.argtypes = [P, P, I64]
        lib.orc_e4m3_encode_array.restype = None
        lib.orc_e4m3_encode_bits.argtypes = [ctypes.c_uint32, I64, P]
        lib.orc_e4m3_encode_bits.restype = None
        lib.orc_f32_to_bf16.argtypes = [ctypes.c_float]
        lib.orc_f32_to_bf16.restype = ctypes.c_uint16
        lib.orc_quantize.argtypes = [P, P, P, I64, I64, I64, I64, ctypes.c_int, P, P, P, P, P, P, P, P]
        lib.orc_quantize.restype = None
        lib.orc_attention_rows.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, ctypes.c_int,
                                           ctypes.c_float, I64, P, P, P, P, P, P, P, P]
        lib.orc_attention_rows.restype = None
        lib.orc_attention.argtypes = [P, P, P, P, P, P, P, P, I64, I64, I64, I64, ctypes.c_int,
                                      ctypes.c_float, P, P]
        lib.orc_attention.restype = None
        lib.orc_attention_sparse.argtypes = [P, P, P, P, P, P, P, P, P, I64, I64, I64, I64, ctypes.c_int,
                                             ctypes.c_float, P, P]
        lib.orc_attention_sparse.restype = None
        lib.orc_bruteforce.argtypes = [P, P, P, I64, I64, I64, I64, ctypes.c_double, P]
        lib.orc_bruteforce.restype = None
        lib.orc_rounding_mode_is_nearest.argtypes = []
        lib.orc_rounding_mode_is_nearest.restype = ctypes.c_int
        lib.orc_num_threads.argtypes = []
        lib.orc_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a)
    assert a.dtype == dtype, (a.dtype, dtype)
    return a


def nblocks(n: int) -> int:
    return (n + BLK - 1) // BLK


# ------------------------------------------------------------------ E4M3 ----
def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    lib = _load()
    table = np.array([lib.orc_e4m3_decode(c) for c in range(256)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    x = _c(np.asarray(x, dtype=np.float32), np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    _load().orc_e4m3_encode_array(x.ctypes.data, out.ctypes.data, x.size)
    return out


def e4m3_encode_nearest(x: float) -> int:
    return int(_load().orc_e4m3_encode_nearest(float(x)))


def e4m3_sweep_mismatches(lo: int, hi: int) -> int:
    return int(_load().orc_e4m3_sweep_mismatches(lo, hi))


def e4m3_encode_bits(lo: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint8)
    _load().orc_e4m3_encode_bits(lo, n, out.ctypes.data)
    return out


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    lib = _load()
    x = np.asarray(x, dtype=np.float32)
    return np.array([lib.orc_f32_to_bf16(float(v)) for v in x.ravel()], dtype=np.uint16).reshape(x.shape)


# -------------------------------------------------------------- quantize ----
QK_FORMATS = {"int8": 0, "fp8": 1}


def quantize(q: np.ndarray, k: np.ndarray, v: np.ndarray, qk_format: str = "int8",
             q_smooth: bool = False) -> Dict[str, np.ndarray]:
    """Codes and scales; qk_format "int8" (scale amax/127) or "fp8" (E4M3
    bit patterns, scale amax/448) for Q and smoothed K.  With q_smooth, Q is
    smoothed per 128-token block (codes of q - block mean) and "q_mean"
    [B, H, nbq, 128] holds the means; the attention functions then add the
    Delta-S term back to every score."""
    fmt = QK_FORMATS[qk_format]
    B, Nq, H, d = q.shape
    Nkv = k.shape[1]
    assert d == D and k.shape == (B, Nkv, H, D) and v.shape == (B, Nkv, H, D)
    q, k, v = (_c(t, np.uint16) for t in (q, k, v))
    qm = np.empty((B, H, nblocks(Nq), D), np.float32) if q_smooth else None
    r = {
        "q8": np.empty((B, H, Nq, D), np.int8),
        "k8": np.empty((B, H, Nkv, D), np.int8),
        "v8": np.empty((B, H, Nkv, D), np.uint8),
        "q_scale": np.empty((B, H, nblocks(Nq)), np.float32),
        "k_scale": np.empty((B, H, nblocks(Nkv)), np.float32),
        "v_scale": np.empty((B, H, D), np.float32),
        "k_mean": np.empty((B, H, D), np.float32),
    }
    _load().orc_quantize(q.ctypes.data, k.ctypes.data, v.ctypes.data, B, H, Nq, Nkv, fmt,
                         *(r[n].ctypes.data for n in ("q8", "k8", "v8", "q_scale", "k_scale",
                                                      "v_scale", "k_mean")),
                         None if qm is None else qm.ctypes.data)
    r["qk_format"] = qk_format
    if q_smooth:
        r["q_mean"] = qm
    return r


def _qmean_ptr(c: Dict[str, np.ndarray]):
    qm = c.get("q_mean")
    return None if qm is None else _c(qm, np.float32)


def _code_args(c: Dict[str, np.ndarray]):
    arrs = [_c(c["q8"], np.int8), _c(c["k8"], np.int8), _c(c["v8"], np.uint8),
            _c(c["q_scale"], np.float32), _c(c["k_scale"], np.float32), _c(c["v_scale"], np.float32)]
    return arrs


# ------------------------------------------------------------- attention ----
def attention(codes: Dict[str, np.ndarray], softmax_scale: float, return_lse: bool = False):
    """Every row; BF16 bits, BSHD [B, Nq, H, 128].  With return_lse, also the
    log-sum-exp of each row's logits before K smoothing, FP64 [B, H, Nq]."""
    B, H, Nq, _ = codes["q8"].shape
    Nkv = codes["k8"].shape[2]
    arrs = _code_args(codes)
    out = np.empty((B, Nq, H, D), np.uint16)
    lse = np.empty((B, H, Nq), np.float64) if return_lse else None
    km = _c(codes["k_mean"], np.float32) if return_lse else None
    qm = _qmean_ptr(codes)
    _load().orc_attention(*(a.ctypes.data for a in arrs), None if km is None else km.ctypes.data,
                          None if qm is None else qm.ctypes.data, B, H, Nq, Nkv, QK_FORMATS[codes.get("qk_format", "int8")], softmax_scale,
                          out.ctypes.data, None if lse is None else lse.ctypes.data)
    return (out, lse) if return_lse else out


def attention_sparse(codes: Dict[str, np.ndarray], softmax_scale: float, block_mask: np.ndarray,
                     return_lse: bool = False):
    """Block-sparse attention: query i attends key j iff
    block_mask[b, h, i // 128, j // 128] (uint8/bool [B, H, nbq, nbk]).  As
    ``attention`` over each row's allowed keys; a row without one gets
    output 0 (and lse -inf)."""
    B, H, Nq, _ = codes["q8"].shape
    Nkv = codes["k8"].shape[2]
    mask = _c(np.asarray(block_mask).astype(np.uint8), np.uint8)
    assert mask.shape == (B, H, nblocks(Nq), nblocks(Nkv)), mask.shape
    arrs = _code_args(codes)
    out = np.empty((B, Nq, H, D), np.uint16)
    lse = np.empty((B, H, Nq), np.float64) if return_lse else None
    km = _c(codes["k_mean"], np.float32) if return_lse else None
    qm = _qmean_ptr(codes)
    _load().orc_attention_sparse(*(a.ctypes.data for a in arrs), None if km is None else km.ctypes.data,
                                 None if qm is None else qm.ctypes.data, mask.ctypes.data, B, H, Nq, Nkv, QK_FORMATS[codes.get("qk_format", "int8")],
                                 softmax_scale, out.ctypes.data, None if lse is None else lse.ctypes.data)
    return (out, lse) if return_lse else out


def attention_rows(codes: Dict[str, np.ndarray], softmax_scale: float,
                   rows: np.ndarray, return_lse: bool = False, block_mask: Optional[np.ndarray] = None):
    """rows: int64 [n, 3] of (b, h, i).  Returns (out BF16 [n,128], m [n], l [n]),
    and lse [n] (as in ``attention``) after them with return_lse.  With a
    block_mask, the rows of ``attention_sparse``."""
    B, H, Nq, _ = codes["q8"].shape
    Nkv = codes["k8"].shape[2]
    rows = _c(np.asarray(rows, dtype=np.int64).reshape(-1, 3), np.int64)
    assert rows.size == 0 or (rows[:, 0].max() < B and rows[:, 1].max() < H and rows[:, 2].max() < Nq
                              and rows.min() >= 0)
    n = rows.shape[0]
    arrs = _code_args(codes)
    out = np.empty((n, D), np.uint16)
    m = np.empty(n, np.float64)
    l = np.empty(n, np.float64)
    lse = np.empty(n, np.float64) if return_lse else None
    km = _c(codes["k_mean"], np.float32) if return_lse else None
    mask = None
    if block_mask is not None:
        mask = _c(np.asarray(block_mask).astype(np.uint8), np.uint8)
        assert mask.shape == (B, H, nblocks(Nq), nblocks(Nkv)), mask.shape
    qm = _qmean_ptr(codes)
    _load().orc_attention_rows(*(a.ctypes.data for a in arrs), B, H, Nq, Nkv,
                               QK_FORMATS[codes.get("qk_format", "int8")], softmax_scale, n,
                               rows.ctypes.data, None if km is None else km.ctypes.data,
                               None if qm is None else qm.ctypes.data,
                               None if mask is None else mask.ctypes.data,
                               out.ctypes.data, m.ctypes.data, l.ctypes.data,
                               None if lse is None else lse.ctypes.data)
    return (out, m, l, lse) if return_lse else (out, m, l)


def bruteforce(q: np.ndarray, k: np.ndarray, v: np.ndarray, softmax_scale: float) -> np.ndarray:
    """Exact softmax(Q K^T scale) V in FP64 from the BF16 inputs; BSHD float64."""
    B, Nq, H, _ = q.shape
    Nkv = k.shape[1]
    q, k, v = (_c(t, np.uint16) for t in (q, k, v))
    out = np.empty((B, Nq, H, D), np.float64)
    _load().orc_bruteforce(q.ctypes.data, k.ctypes.data, v.ctypes.data, B, H, Nq, Nkv,
                           float(softmax_scale), out.ctypes.data)
    return out


def rounding_mode_is_nearest() -> bool:
    return bool(_load().orc_rounding_mode_is_nearest())


def num_threads() -> int:
    """Threads the oracle's OpenMP regions use."""
    return int(_load().orc_num_threads())
