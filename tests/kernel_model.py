"""A CPU model of the attention kernel's FP32 arithmetic -- test tooling.

The oracle defines what the method computes: a two-pass softmax whose P
codes are E4M3(448 p) against each row's final maximum.  The kernel runs an
online softmax instead (one pass over key tiles, P quantised against the
running maximum, O and l rescaled when the maximum grows).  That is a
different rounding of the same quantity, and only the outputs are compared.
This module models the kernel's online form step by step in numpy, from the
oracle's codes, so that the size of that difference can be measured on the
CPU for any scale, shape and seed:

  per row and key tile (``tile`` keys, within one 128-key quantisation block)
    c     = fl32(fl32(qs * ks) * fl32(softmax_scale * log2 e))
    mt    = fl32(max_j acc_j * c)          (integer max; c > 0)
    mnew  = max(m, mt); alpha = fl32(2^(m - mnew)); O, l *= alpha
    t_j   = fl32(acc_j * c + fl32(log2 448 - mnew))     (one FMA)
    p_j   = fl32(2^t_j)   (448 p, as P is scaled by 448)
    l    += sum_j p_j (FP32);  O += E4M3(p_j) . V8_j
  out = bf16(fl32(fl32(O * vs) / l)).

``fold=True`` models the earlier kernel form that read the INT8
accumulators as floats carrying the bias 1.5 * 2^23 and folded that bias into
the exponent constant, fl32(log2 448 - mnew - 1.5 * 2^23 * c), rounded once
per row and tile.

Nothing here is an oracle: the GPU tests compare the kernel with the oracle.
This model explains and bounds the kernel-side part of that difference
(used by tests/test_kernel_model.py)."""
import numpy as np

import oracle

LOG2E = np.float32(1.4426950408889634)
LOG2_448 = np.float32(np.log2(448.0))
MAGIC = np.float32(12582912.0)  # 1.5 * 2^23


def _f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def _decode(codes):
    return oracle.e4m3_decode(codes)


def _bf16(x):
    """FP32 -> BF16 bits, round to nearest even (finite values)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def online_attention(codes, softmax_scale: float, tile: int = 128, fold: bool = False,
                     split: int = 1) -> np.ndarray:
    """BF16 bits [B, Nq, H, 128] of the kernel's online softmax (INT8 Q/K).

    tile: keys per step (64 or 128; within one 128-key block).  split: key
    ranges of whole 128-key blocks, merged by the LSE rule in FP32 (the
    split-KV path), 1 for none."""
    assert codes.get("qk_format", "int8") == "int8"
    assert 128 % tile == 0
    q8, k8, v8 = codes["q8"], codes["k8"], codes["v8"]
    B, H, Nq, _ = q8.shape
    Nkv = k8.shape[2]
    nbk = -(-Nkv // 128)
    sl2e = _f32(np.float32(softmax_scale) * LOG2E)
    out = np.empty((B, Nq, H, 128), np.uint16)
    tps = -(-nbk // split)
    for b in range(B):
        for h in range(H):
            acc = q8[b, h].astype(np.int64) @ k8[b, h].astype(np.int64).T       # [Nq, Nkv]
            vd = _decode(v8[b, h])                                            # [Nkv, 128]
            qs = codes["q_scale"][b, h][np.arange(Nq) // 128].astype(np.float32)
            ks = codes["k_scale"][b, h].astype(np.float32)
            vs = codes["v_scale"][b, h].astype(np.float32)
            parts = []
            for s0 in range(0, nbk, tps):
                m = np.full(Nq, -np.inf, np.float32)
                l = np.zeros(Nq, np.float32)
                O = np.zeros((Nq, 128), np.float64)
                first = True
                for j0 in range(s0 * 128, min(nbk, s0 + tps) * 128, tile):
                    j1 = min(j0 + tile, Nkv)
                    if j1 <= j0:
                        break
                    c = _f32(_f32(qs * ks[j0 // 128]) * sl2e)                 # [Nq]
                    c = np.where(c == 0, np.float32(1.17549435e-38), c)
                    a = acc[:, j0:j1]
                    mt = _f32(a.max(axis=1).astype(np.float64) * c.astype(np.float64))
                    mnew = np.maximum(m, mt)
                    if not first:
                        alpha = _f32(np.exp2((m - mnew).astype(np.float64)))
                        l = _f32(l * alpha)
                        O = _f32(O * alpha[:, None]).astype(np.float64)
                    first = False
                    m = mnew
                    if fold:
                        nb = _f32(_f32(LOG2_448 - mnew).astype(np.float64)
                                  - np.float64(MAGIC) * c.astype(np.float64))
                        sf = (a + 12582912).astype(np.float64)
                        t = _f32(sf * c[:, None].astype(np.float64) + nb[:, None].astype(np.float64))
                    else:
                        nb = _f32(LOG2_448 - mnew)
                        t = _f32(a.astype(np.float64) * c[:, None].astype(np.float64)
                                 + nb[:, None].astype(np.float64))
                    p = _f32(np.exp2(t.astype(np.float64)))
                    l = _f32(l + p.sum(axis=1, dtype=np.float32))
                    p8 = _decode(oracle.e4m3_encode(p))
                    O = _f32(O + p8 @ vd[j0:j1]).astype(np.float64)
                parts.append((m, l, O))
            if len(parts) == 1:
                m, l, O = parts[0]
                o = _f32(_f32(O * vs[None, :]) * _f32(np.float32(1.0) / l)[:, None])
            else:
                # each range: normalised FP32 output and lse (log2 units here)
                lse = [p_[0].astype(np.float64) + np.log2(p_[1].astype(np.float64)) - float(LOG2_448)
                       for p_ in parts]
                outs = [_f32(_f32(p_[2] * vs[None, :]) * _f32(np.float32(1.0) / p_[1])[:, None])
                        for p_ in parts]
                mx = np.max(np.stack(lse), axis=0)
                w = [_f32(np.exp2(x - mx)) for x in lse]
                wsum = _f32(sum(w))
                acc_o = sum(w_[:, None].astype(np.float64) * o_ for w_, o_ in zip(w, outs))
                o = _f32(_f32(acc_o) * _f32(np.float32(1.0) / wsum)[:, None])
            out[b, :, h, :] = _bf16(o)
    return out
