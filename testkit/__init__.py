"""Seeded synthetic inputs for the attention tests and benchmark.

This module holds none of the method's arithmetic.  It draws BF16 Q/K/V of
shape [B, N, H, 128] (BSHD) with the value structure of diffusion-transformer
attention (Gaussian activations, a per-(head, channel) key bias shared by all
tokens and batch items, one outlier channel per head, heavy tails), using the
counter-based SplitMix64 generator in sattn_testkit.c.  The five workloads
mirror the pages' DiT shapes: a Flux-like joint image+text sequence, Wan-like
video self-attention with a ragged 32760-token tail, text cross-attention
against 512 keys, and the 65520-token standalone length of the FA4 benchmark
("VisualGen FA4 autotuning ...", Validation).
"""
import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# SATTN_TESTKIT_LIB: another build of sattn_testkit.c (the sanitizer test's)
_LIB_PATH = os.environ.get("SATTN_TESTKIT_LIB") or os.path.join(HERE, "libsattn_testkit.so")
_lib = None

STREAM_Q, STREAM_K, STREAM_V, STREAM_KBIAS, STREAM_OUTLIER = 1, 2, 3, 4, 5
NORMAL, STUDENT4 = 0, 1
D = 128


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.tk_fill.argtypes = [ctypes.c_void_p] + [ctypes.c_int64] * 4 + [
            ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int, ctypes.c_double, ctypes.c_uint64,
            ctypes.c_double, ctypes.c_uint64]
        lib.tk_fill.restype = None
        lib.tk_word_export.argtypes = [ctypes.c_uint64] * 4
        lib.tk_word_export.restype = ctypes.c_uint64
        lib.tk_d_to_bf16.argtypes = [ctypes.c_double]
        lib.tk_d_to_bf16.restype = ctypes.c_uint16
        _lib = lib
    return _lib


def word(seed: int, stream: int, index: int, j: int) -> int:
    return int(_load().tk_word_export(seed, stream, index, j))


def d_to_bf16(x: float) -> int:
    return int(_load().tk_d_to_bf16(float(x)))


def fill(B: int, N: int, H: int, seed: int, stream: int, dist: int = NORMAL,
         bias_sigma: float = 0.0, outlier_mult: float = 1.0,
         out: Optional[np.ndarray] = None) -> np.ndarray:
    """BF16 bit patterns, uint16 [B, N, H, 128]."""
    if out is None:
        out = np.empty((B, N, H, D), dtype=np.uint16)
    assert out.dtype == np.uint16 and out.shape == (B, N, H, D) and out.flags.c_contiguous
    assert B < 256 and H < 4096 and N < (1 << 25), "outside the generator's index range"
    _load().tk_fill(out.ctypes.data, B, N, H, D, seed, stream, dist, bias_sigma, STREAM_KBIAS,
                    outlier_mult, STREAM_OUTLIER)
    return out


@dataclass(frozen=True)
class Config:
    index: int
    name: str
    B: int
    H: int
    Nq: int
    Nkv: int
    q_dist: int = NORMAL
    k_dist: int = NORMAL
    k_bias: float = 0.0
    outlier: float = 1.0
    cross: bool = False
    density: Optional[float] = None  # block-sparse: block_mask density (None: dense)

    @property
    def seed(self) -> int:
        return 42 + self.index

    @property
    def flops(self) -> int:
        """4 * (query, key) pairs attended * D: all pairs, or those the
        workload's block mask allows."""
        if self.density is None:
            return 4 * self.B * self.H * self.Nq * self.Nkv * D
        m = self.block_mask().astype(np.int64)
        rows = np.minimum(128, self.Nq - 128 * np.arange(m.shape[2]))
        keys = np.minimum(128, self.Nkv - 128 * np.arange(m.shape[3]))
        return int(4 * D * np.einsum("bhqk,q,k->", m, rows, keys))

    def block_mask(self) -> np.ndarray:
        return block_mask(self.B, self.H, self.Nq, self.Nkv, self.density, seed=self.seed)

    @property
    def softmax_scale(self) -> float:
        return 1.0 / np.sqrt(128.0)

    def describe(self) -> dict:
        d = {"workload": self.name, "B": self.B, "H": self.H, "Nq": self.Nq, "Nkv": self.Nkv,
             "D": D, "seed": self.seed}
        if self.density is not None:
            d["block_density"] = self.density
        return d


CONFIGS = {
    1: Config(1, "tiny self-attention", 1, 2, 256, 256),
    2: Config(2, "flux-like joint image+text self-attention", 1, 24, 4608, 4608, k_bias=2.0),
    3: Config(3, "text cross-attention", 2, 40, 32760, 512, k_bias=1.0, cross=True),
    4: Config(4, "wan-like video self-attention", 1, 40, 32760, 32760, k_bias=2.0, outlier=8.0),
    5: Config(5, "long-sequence self-attention", 1, 24, 65520, 65520, q_dist=STUDENT4,
              k_dist=STUDENT4, k_bias=3.0),
    # few queries against the Wan-like keys: 40 workgroups without split-KV
    6: Config(6, "short-query long-key attention", 1, 40, 256, 32760, k_bias=2.0, outlier=8.0,
              cross=True),
    # the Wan-like workload under a seeded block mask keeping half the blocks
    7: Config(7, "wan-like video block-sparse attention", 1, 40, 32760, 32760, k_bias=2.0,
              outlier=8.0, density=0.5),
}


def make_inputs(cfg: Config, seed: Optional[int] = None, B: Optional[int] = None,
                H: Optional[int] = None, Nq: Optional[int] = None,
                Nkv: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Q, K, V for a workload; shape overrides keep its value recipe."""
    s = cfg.seed if seed is None else seed
    B = cfg.B if B is None else B
    H = cfg.H if H is None else H
    Nq = cfg.Nq if Nq is None else Nq
    Nkv = cfg.Nkv if Nkv is None else Nkv
    q = fill(B, Nq, H, s, STREAM_Q, cfg.q_dist, 0.0, cfg.outlier)
    k = fill(B, Nkv, H, s, STREAM_K, cfg.k_dist, cfg.k_bias, cfg.outlier)
    v = fill(B, Nkv, H, s, STREAM_V, NORMAL, 0.0, cfg.outlier)
    return q, k, v


def block_mask(B: int, H: int, Nq: int, Nkv: int, density: float, seed: int,
               keep_diagonal: bool = True) -> np.ndarray:
    """Seeded block-sparse pattern, uint8 [B, H, ceil(Nq/128), ceil(Nkv/128)]:
    each (query block, key block) pair kept with probability `density`, and
    (with keep_diagonal) the pairs on the block diagonal always, as a local
    window would.  Drawn with numpy's PCG64 from `seed`."""
    nbq, nbk = -(-Nq // 128), -(-Nkv // 128)
    m = (np.random.default_rng(seed).random((B, H, nbq, nbk)) < density).astype(np.uint8)
    if keep_diagonal:
        d = np.arange(min(nbq, nbk))
        m[:, :, d, d] = 1
    return m


def bf16_to_f32(x: np.ndarray) -> np.ndarray:
    """Exact widening of BF16 bit patterns."""
    return (x.astype(np.uint32) << 16).view(np.float32)
