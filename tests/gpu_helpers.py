"""Shared helpers for the GPU parity tests: seeded inputs on the device, the
oracle's codes and outputs for the same inputs, and the parity metrics."""
import functools
import sys
import time

import numpy as np

import fp8_mfma_model
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


def sample_rows_strided(B: int, H: int, Nq: int, stride: int, seed: int) -> np.ndarray:
    """One row in every `stride` consecutive query rows of every (b, h), at a
    seeded offset inside the group, plus each head's first and last row and
    the rows around its last full 128-row block.  With stride 32 every wave's
    32 queries are represented (and so every workgroup, query tile and
    position of the workgroup-to-XCD mapping)."""
    rng = np.random.default_rng(seed)
    starts = np.arange(0, Nq, stride)
    rows = []
    for b in range(B):
        for h in range(H):
            off = rng.integers(0, stride, size=starts.size)
            idx = np.minimum(starts + off, Nq - 1)
            extra = [0, Nq - 1, max(0, Nq - 129)]
            if (Nq // 128) * 128 < Nq:
                extra.append((Nq // 128) * 128)
            idx = np.unique(np.concatenate([idx, np.array(extra, dtype=np.int64)]))
            rows.append(np.stack([np.full(idx.size, b), np.full(idx.size, h), idx], axis=1))
    return np.concatenate(rows).astype(np.int64)


# rows per sample group at full size: every wave of the Wan-like and
# cross-attention workloads; on the long-sequence one (whose oracle rows
# cost twice as much) one row in every 128, i.e. every query block
FULL_SIZE_STRIDE = {3: 32, 4: 32, 5: 128}


# FP8 Q/K format: v_mfma_scale_f32_32x32x64_f8f6f4 does not return the
# correctly rounded sum of its products (the INT8 instruction is exact).
# fp8_mfma_model states how it sums them and bounds the score error per
# (query, key) from the codes; a score error of at most delta_i (natural-log
# units) on row i moves that row's output by at most 2 delta_i max|V| to
# first order.
def fp8_score_error(codes, scale, rows=None) -> np.ndarray:
    """delta per query row: max_j of the model's dot-product error bound for
    (q_i, k_j) in code units, times qs_i ks_j softmax_scale, from the
    oracle's codes.  [B, H, Nq], or [n] for rows[:, (b, h, i)].  The bound,
    TRUNC_REL * G + SUM_REL * S, comes out of one matrix product of the
    rows' scaled code magnitudes and group weights, side by side, with the
    keys' (buffers allocated once per call)."""
    B, H, Nq, _ = codes["q8"].shape
    Nkv = codes["k8"].shape[2]
    out = np.zeros((B, H, Nq)) if rows is None else np.zeros(len(rows))
    step = 2048
    ng = 128 // fp8_mfma_model.GROUP
    kwT = np.empty((128 + ng, Nkv))
    e = None
    for b in range(B):
        for h in range(H):
            if rows is None:
                qi = np.arange(Nq)
                sel = None
            else:
                sel = np.nonzero((rows[:, 0] == b) & (rows[:, 1] == h))[0]
                if sel.size == 0:
                    continue
                qi = rows[sel, 2]
            qc = codes["q8"][b, h, qi].view(np.uint8)
            kc = codes["k8"][b, h].view(np.uint8)
            ks = codes["k_scale"][b, h][np.arange(Nkv) // 128].astype(np.float64)
            qw = np.concatenate([np.abs(fp8_mfma_model.e4m3_value(qc)) * fp8_mfma_model.SUM_REL,
                                 fp8_mfma_model.group_weights(qc) * fp8_mfma_model.TRUNC_REL], axis=1)
            np.take(fp8_mfma_model.e4m3_magnitudes(), kc.T, out=kwT[:128])
            kwT[128:] = fp8_mfma_model.group_weights(kc).T
            kwT *= ks[None, :]
            n = len(qi)
            if e is None or e.shape[0] < n:
                e = np.empty((n, step))
            worst = np.zeros(n)
            for j0 in range(0, Nkv, step):
                j1 = min(Nkv, j0 + step)
                np.matmul(qw, kwT[:, j0:j1], out=e[:n, :j1 - j0])
                np.maximum(worst, e[:n, :j1 - j0].max(axis=1), out=worst)
            d = worst * codes["q_scale"][b, h][qi // 128].astype(np.float64) * scale
            if sel is None:
                out[b, h] = d
            else:
                out[sel] = d
    return out


def out_bar(codes, scale, rows=None):
    """Per-row bar on max_d |O_gpu - O_oracle| / max|V|: 2e-2, plus 2 delta_i
    in the FP8 Q/K format.  [B, H, Nq], or [n] for rows."""
    if codes.get("qk_format", "int8") != "fp8":
        B, H, Nq, _ = codes["q8"].shape
        return np.full((B, H, Nq) if rows is None else (len(rows),), MAX_ERR)
    return MAX_ERR + 2.0 * fp8_score_error(codes, scale, rows)


def row_errors(o_gpu_bits: np.ndarray, o_orc_bits: np.ndarray, max_abs_v: float) -> np.ndarray:
    """max_d |O_gpu - O_oracle| / max|V| per row: [B, H, Nq] from BSHD
    outputs, or [n] from [n, 128] rows."""
    a = testkit.bf16_to_f32(o_gpu_bits).astype(np.float64)
    b = testkit.bf16_to_f32(o_orc_bits).astype(np.float64)
    e = np.abs(a - b).max(axis=-1) / max_abs_v
    return np.transpose(e, (0, 2, 1)) if e.ndim == 3 else e


def check_rows(o_gpu_bits, o_orc_bits, v_bits, bar_rows, what, min_cos=MIN_COS):
    """Every row within its bar and the global cosine >= min_cos; returns
    (worst error / bar, max error, cosine)."""
    mv = float(np.abs(testkit.bf16_to_f32(v_bits)).max())
    e = row_errors(o_gpu_bits, o_orc_bits, mv)
    _, c = parity(o_gpu_bits, o_orc_bits, mv)
    ratio = float(np.max(e / bar_rows)) if e.size else 0.0
    log(f"  {what}: max err / max|V| = {float(e.max()):.3e}, worst err / bar = {ratio:.3f} "
        f"(bar {float(np.min(bar_rows)):.2e}..{float(np.max(bar_rows)):.2e}), cos = {c:.7f}")
    assert ratio <= 1.0 and c >= min_cos, (ratio, c)
    return ratio, float(e.max()), c


def smooth_units(codes):
    """With Q smoothing and INT8 codes the kernel counts each block's scores
    in a unit of its own: qs, or qs 2^k with
    k = max(0, ilogb(amax|qmean|) - ilogb(qs) - 14) when the mean exceeds
    2^15 code units (the kernel then rounds the codes to multiples of 2^k),
    or amax|qmean| 2^-14 (at least the smallest normal float; 1 for a zero
    mean) when qs = 0.  Returns (unit, k), each [B, H, nbq], the units as the
    kernel's FP32 values."""
    qs = codes["q_scale"].astype(np.float32)
    amax = np.abs(codes["q_mean"].astype(np.float32)).max(axis=-1)
    ilogb = lambda x: np.frexp(x)[1].astype(np.int64) - 1  # noqa: E731
    pos = qs > 0
    k = np.where(pos & (amax > 0), np.maximum(0, ilogb(np.where(amax > 0, amax, 1))
                                              - ilogb(np.where(pos, qs, 1)) - 14), 0)
    zero_unit = np.where(amax > 0, np.maximum(np.ldexp(amax, -14).astype(np.float32),
                                              np.float32(1.17549435e-38)), np.float32(1.0))
    unit = np.where(pos, np.ldexp(qs, k).astype(np.float32), zero_unit).astype(np.float32)
    return unit.astype(np.float64), k


def lse_bar(codes, scale, rows=None) -> np.ndarray:
    """Per-row bar on |lse_gpu - lse_oracle| (natural log), derived from the
    kernel's FP32 steps (u = 2^-24):
      - the dequantisation constant c = fl(fl(qs ks) fl(scale log2 e)) and
        the row maximum m = fl(acc c) carry <= 5u relative error, and with
        Q smoothing the FP32 sums acc + Delta-S and the Delta-S products
        <= 129u: 2^-17 * smag, smag = max_j sum_d q~_id |k~_jd| * scale;
      - the K-mean shift, a 64-term FMA chain per lane plus one add:
        2^-17 * sum_d q~_id |kmean_d| * scale;
      - the FP32 row sum of at most Nkv positive terms, rescaled at most
        once per key tile by an exp2 within 2u: (Nkv + 2 nbk) u;
      - log2, exp2 and the final operations: 2^-20;
    with q~ = |qcode| qs (+ |qmean| with Q smoothing) and k~ = |kcode| ks.
    The FP8 Q/K format adds the row's delta (fp8_score_error).  With Q
    smoothing and INT8 codes, Delta-S is rounded to the block's unit (see
    smooth_units) after a four-digit expansion of qmean / unit (digits below
    2^-27 amax|qmean| dropped): + (0.5 unit max_j ks_j + 2^-27 amax|qmean|
    sk) * scale, sk = max_j sum_d |kcode_jd| ks_j; where the codes were
    rounded to multiples of 2^k, each moved by at most r = min(unit / 2,
    127 qs): + r (sk + sum_d |kmean_d|) * scale.  [B, H, Nq], or [n] for
    rows."""
    fmt = codes.get("qk_format", "int8")
    B, H, Nq, _ = codes["q8"].shape
    Nkv = codes["k8"].shape[2]
    nbk = -(-Nkv // 128)
    dec = ((lambda c: np.abs(oracle.e4m3_decode(c.view(np.uint8)))) if fmt == "fp8"
           else (lambda c: np.abs(c.astype(np.float64))))
    out = np.zeros((B, H, Nq)) if rows is None else np.zeros(len(rows))
    units = smooth_units(codes) if fmt != "fp8" and "q_mean" in codes else None
    for b in range(B):
        for h in range(H):
            if rows is None:
                qi, sel = np.arange(Nq), None
            else:
                sel = np.nonzero((rows[:, 0] == b) & (rows[:, 1] == h))[0]
                if sel.size == 0:
                    continue
                qi = rows[sel, 2]
            qt = dec(codes["q8"][b, h, qi]) * codes["q_scale"][b, h][qi // 128].astype(np.float64)[:, None]
            if "q_mean" in codes:
                qt = qt + np.abs(codes["q_mean"][b, h][qi // 128].astype(np.float64))
            kt = dec(codes["k8"][b, h]) * codes["k_scale"][b, h][np.arange(Nkv) // 128].astype(np.float64)[:, None]
            smag = np.zeros(len(qi))
            for j0 in range(0, Nkv, 8192):
                smag = np.maximum(smag, (qt @ np.ascontiguousarray(kt[j0:j0 + 8192].T)).max(axis=1))
            shift = qt @ np.abs(codes["k_mean"][b, h].astype(np.float64))
            bar = 2.0 ** -17 * (smag + shift) * scale + (Nkv + 2 * nbk) * 2.0 ** -24 + 2.0 ** -20
            if fmt != "fp8" and "q_mean" in codes:
                unit, ksh = units[0][b, h][qi // 128], units[1][b, h][qi // 128]
                ks = codes["k_scale"][b, h].astype(np.float64)
                sk = (np.abs(codes["k8"][b, h].astype(np.float64)).sum(axis=1) * ks[np.arange(Nkv) // 128]).max()
                amq = np.abs(codes["q_mean"][b, h][qi // 128].astype(np.float64)).max(axis=1)
                qsr = codes["q_scale"][b, h][qi // 128].astype(np.float64)
                r = np.where(ksh > 0, np.minimum(0.5 * unit, 127.0 * qsr), 0.0)
                kms = np.abs(codes["k_mean"][b, h].astype(np.float64)).sum()
                bar = bar + (0.5 * unit * ks.max() + 2.0 ** -27 * amq * sk + r * (sk + kms)) * scale
            if sel is None:
                out[b, h] = bar
            else:
                out[sel] = bar
    if fmt == "fp8":
        out = out + fp8_score_error(codes, scale, rows)
    return out
