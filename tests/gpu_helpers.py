"""Shared helpers for the GPU parity tests: seeded inputs on the device, the
oracle's codes and outputs for the same inputs, and the parity metrics."""
import functools
import sys
import time

import numpy as np

import oracle
import testkit


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(bits: np.ndarray):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to("cuda:0")


def from_dev(t) -> np.ndarray:
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@functools.lru_cache(maxsize=1)
def workload(cfg_index: int):
    """(cfg, q, k, v, oracle codes) at the full size of a workload."""
    cfg = testkit.CONFIGS[cfg_index]
    t0 = time.time()
    q, k, v = testkit.make_inputs(cfg)
    t1 = time.time()
    codes = oracle.quantize(q, k, v)
    log(f"  [{cfg.name}] inputs {t1 - t0:.1f}s, oracle quantize {time.time() - t1:.1f}s")
    return cfg, q, k, v, codes


CODE_KEYS = ("q8", "k8", "v8", "q_scale", "k_scale", "v_scale", "k_mean")


def assert_codes_equal(got, want):
    for n in CODE_KEYS:
        a, b = got[n], want[n]
        assert a.shape == b.shape, (n, a.shape, b.shape)
        if a.dtype == np.float32:
            same = a.view(np.uint32) == b.view(np.uint32)
        else:
            same = a == b
        if not np.all(same):
            idx = np.argwhere(~same)[:5]
            raise AssertionError(f"{n}: {int((~same).sum())} of {a.size} differ; first at {idx.tolist()}: "
                                 f"got {[a[tuple(i)] for i in idx]} want {[b[tuple(i)] for i in idx]}")


def parity(o_gpu_bits: np.ndarray, o_orc_bits: np.ndarray, max_abs_v: float):
    """(max abs error / max|V|, global cosine) in FP64."""
    a = testkit.bf16_to_f32(o_gpu_bits).astype(np.float64).ravel()
    b = testkit.bf16_to_f32(o_orc_bits).astype(np.float64).ravel()
    err = float(np.abs(a - b).max()) / max_abs_v
    c = float(a @ b / np.sqrt((a @ a) * (b @ b)))
    return err, c


MAX_ERR = 2e-2   # max |O_gpu - O_oracle| / max|V|
MIN_COS = 0.9995


def sample_rows(B: int, H: int, Nq: int, per_head: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    rows = []
    for b in range(B):
        for h in range(H):
            idx = set(rng.integers(0, Nq, size=per_head).tolist())
            idx.update({0, Nq - 1, max(0, Nq - 129), (Nq // 128) * 128 if (Nq // 128) * 128 < Nq else 0})
            rows.extend((b, h, i) for i in sorted(idx))
    return np.array(rows, dtype=np.int64)
