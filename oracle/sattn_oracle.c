/*
 * sattn_oracle.c -- plain, slow, CPU reference for the INT8-QK / FP8-PV
 * attention forward.  TEST INFRASTRUCTURE ONLY: nothing in the product
 * library links, loads or calls this file; only the test suite, the smoke
 * check and the CPU-baseline leg of the benchmark use it.
 *
 * What it computes follows the pages' problem statement:
 *   - "[ROCm] Add aiter_sage_attn attention backend for gfx1201 (RDNA4)",
 *     section "Changes": INT8 Q.K^T, FP8 P.V, FP32 accumulation, BF16 Q/K/V,
 *     head dim 128, non-causal, softmax_scale passed through.
 *   - "new MHA v4 entrypoint ...", section "Technical Details" and the
 *     throughput table: INT8 Q/K with FP8 V and BF16 output; the lint-bot
 *     import listing names a two-stage per-channel V amax (partial, then
 *     finalize, then quantize) and a log2(e) constant for an exp2 softmax.
 * The quantizer details that the pages leave open (block size, smoothing,
 * rounding, P scaling) are fixed by the method definition this library
 * implements: per-128-token-block INT8 for Q and mean-smoothed K with scale
 * amax/127 and round-half-even, per-(batch, head, channel) OCP E4M3 for V with
 * scale amax/448, P scaled by 448 and rounded to E4M3, the row sum taken from
 * FP32 P, and a full two-pass softmax.
 * A second Q/K format (ORC_QK_FP8) follows the FP8/FP8/BF16 row of the MHA v4
 * page's MI355X throughput table: Q and mean-smoothed K as OCP E4M3 with
 * per-block scale amax/448 (the same encoder and clamp as V), and exact
 * FP64 dot products of the decoded codes.
 *
 * The attention entry points can also return each row's log-sum-exp (the
 * float32 LSE kept beside the output in the FA4 autotuning page,
 * "Validation"): that of the logits before K smoothing, i.e. the row's
 * m + ln(l) plus the logit shift the smoothing removed.
 *
 * Every loop runs in index order.  FP32 steps are single IEEE operations;
 * this file must be compiled with -ffp-contract=off and without fast-math.
 * Layouts: BF16 inputs are BSHD [B][N][H][128] contiguous (uint16 bit
 * patterns); codes are canonical [B][H][N][128]; scales [B][H][nblocks] and
 * [B][H][128].
 */
#include <stdint.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>
#include <fenv.h>
#include <omp.h>

#define D 128
#define BLK 128

/* ---------------------------------------------------------------- BF16 --- */

/* BF16 -> FP32 is exact: the 16 bits become the top half of the FP32 word. */
static float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* FP32 -> BF16 round-to-nearest-even (finite inputs). */
uint16_t orc_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

/* ---------------------------------------------------------- OCP E4M3 ------ */
/*
 * OCP 8-bit floating point, E4M3 variant: 1 sign bit, 4 exponent bits with
 * bias 7, 3 mantissa bits.  Exponent field 0 encodes subnormals m * 2^-9;
 * S.1111.111 is NaN; the largest finite magnitude is S.1111.110 = 448.
 */
double orc_e4m3_decode(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) v = ldexp((double)m, -9);
  else v = ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

/*
 * Arithmetic encoder, round to nearest, ties to the even mantissa.  Input must
 * be finite with |x| <= 448 (callers clamp first).  The sign of zero is kept.
 * Scaling by powers of two is exact in double, so the only rounding is the
 * single nearbyint() under FE_TONEAREST.
 */
uint8_t orc_e4m3_encode(float x) {
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  double a = fabs((double)x);
  if (a == 0.0) return sign;
  if (a < ldexp(1.0, -6)) {
    /* subnormal range: value = m * 2^-9, m in [0, 8]; m == 8 is 2^-6,
       whose code (exponent 1, mantissa 0) is again 8. */
    double m = nearbyint(ldexp(a, 9));
    return (uint8_t)(sign | (uint8_t)m);
  }
  int e2;
  frexp(a, &e2);          /* a = f * 2^e2, f in [0.5, 1) */
  int e = e2 - 1;         /* a in [2^e, 2^(e+1)) */
  double q = nearbyint(ldexp(a, 3 - e)); /* in [8, 16] */
  if (q == 16.0) { q = 8.0; e += 1; }
  int field = e + 7;      /* 1..15 for |x| <= 448 */
  return (uint8_t)(sign | (uint8_t)(field << 3) | (uint8_t)((int)q - 8));
}

/*
 * Independent encoder for the self-check: the nearest of the finite codes of
 * the same sign as x (zero of that sign included), ties to the even code.
 * Because codes are monotone in magnitude, the even code is the one with the
 * even mantissa.
 */
uint8_t orc_e4m3_encode_nearest(float x) {
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  double a = fabs((double)x);
  int best = 0;
  double bestd = INFINITY;
  for (int c = 0; c <= 0x7E; c++) {
    double v = orc_e4m3_decode((uint8_t)c);
    double d = fabs(v - a);
    if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
      bestd = d;
      best = c;
    }
  }
  return (uint8_t)(sign | best);
}

/* Codes of all 32-bit patterns in [lo, hi) whose float is finite with
   |x| <= 448; returns how many differ between the two encoders. */
int64_t orc_e4m3_sweep_mismatches(uint32_t lo, uint32_t hi) {
  /* the nearest-search over a sorted table is fast enough for a sweep */
  double tab[127];
  for (int c = 0; c <= 0x7E; c++) tab[c] = orc_e4m3_decode((uint8_t)c);
  int64_t bad = 0;
  #pragma omp parallel for reduction(+:bad) schedule(static)
  for (int64_t i = (int64_t)lo; i < (int64_t)hi; i++) {
    uint32_t u = (uint32_t)i;
    float x;
    memcpy(&x, &u, 4);
    if (!(fabsf(x) <= 448.0f)) continue;
    double a = fabs((double)x);
    int l = 0, h = 126;      /* largest c with tab[c] <= a */
    while (l < h) { int mid = (l + h + 1) / 2; if (tab[mid] <= a) l = mid; else h = mid - 1; }
    int c = l;
    if (c < 126) {
      double dl = a - tab[c], dh = tab[c + 1] - a;
      if (dh < dl || (dh == dl && (c & 1))) c = c + 1;
    }
    uint8_t ref = (uint8_t)((signbit(x) ? 0x80 : 0) | c);
    if (ref != orc_e4m3_encode(x)) bad++;
  }
  return bad;
}

/* Encode an array (used to produce expected codes for hardware sweeps). */
void orc_e4m3_encode_array(const float* x, uint8_t* out, int64_t n) {
  #pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; i++) out[i] = orc_e4m3_encode(x[i]);
}

/* Encode the floats with bit patterns lo..lo+n-1 (no input array needed). */
void orc_e4m3_encode_bits(uint32_t lo, int64_t n, uint8_t* out) {
  #pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; i++) {
    uint32_t u = lo + (uint32_t)i;
    float x;
    memcpy(&x, &u, 4);
    out[i] = orc_e4m3_encode(x);
  }
}

/* --------------------------------------------------------------- INT8 ----- */

/* code = clamp(RNE(x / s), -127, 127); s == 0 gives 0. */
static int8_t int8_code(float x, float s) {
  if (s == 0.0f) return 0;
  float y = x / s;             /* one correctly rounded FP32 division */
  float r = nearbyintf(y);     /* FE_TONEAREST: ties to even */
  if (r > 127.0f) r = 127.0f;
  if (r < -127.0f) r = -127.0f;
  return (int8_t)r;
}

/* E4M3(clamp(x / s, -448, 448)); s == 0 gives 0x00. */
static uint8_t e4m3_code(float x, float s) {
  if (s == 0.0f) return 0x00;
  float y = x / s;             /* one correctly rounded FP32 division */
  if (y > 448.0f) y = 448.0f;
  if (y < -448.0f) y = -448.0f;
  return orc_e4m3_encode(y);
}

/*
 * Q/K code formats: ORC_QK_INT8 (scale amax/127, INT8 codes) and
 * ORC_QK_FP8 (scale amax/448, OCP E4M3 codes stored as their bit patterns).
 */
enum { ORC_QK_INT8 = 0, ORC_QK_FP8 = 1 };
static float qk_max(int fmt) { return fmt == ORC_QK_FP8 ? 448.0f : 127.0f; }
static int8_t qk_code(float x, float s, int fmt) {
  return fmt == ORC_QK_FP8 ? (int8_t)e4m3_code(x, s) : int8_code(x, s);
}

/* ------------------------------------------------------------ quantize ---- */

static int64_t nblocks(int64_t n) { return (n + BLK - 1) / BLK; }

/*
 * Per (b, h): Q codes per 128-token block; K mean over the sequence (FP32,
 * block partial sums in token order, then the partials in block order, then
 * one division by Nkv); K' = fl32(k - mean) kept in FP32; K' codes per block;
 * V scale per channel = amax/448 and E4M3 codes of clamp(v/s, +-448).
 * Padding rows (tail of the last block) do not exist in the canonical
 * outputs: they hold exactly N rows.
 */
void orc_quantize(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                  int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int fmt,
                  int8_t* q8, int8_t* k8, uint8_t* v8,
                  float* q_scale, float* k_scale, float* v_scale, float* k_mean,
                  float* q_mean) {
  const int64_t nbq = nblocks(Nq), nbk = nblocks(Nkv);
  #pragma omp parallel for collapse(2) schedule(dynamic)
  for (int64_t b = 0; b < B; b++) {
    for (int64_t h = 0; h < H; h++) {
      const int64_t bh = b * H + h;
      /* --- Q (with q_mean: smoothed per block, q' = fl32(q - block mean)) --- */
      for (int64_t t = 0; t < nbq; t++) {
        int64_t n0 = t * BLK, n1 = n0 + BLK < Nq ? n0 + BLK : Nq;
        float qm[D];
        for (int d = 0; d < D; d++) {
          qm[d] = 0.0f;
          if (q_mean) {
            float tot = 0.0f;
            for (int64_t n = n0; n < n1; n++) tot = tot + bf16_to_f32(q[((b * Nq + n) * H + h) * D + d]);
            qm[d] = tot / (float)(n1 - n0);
            q_mean[(bh * nbq + t) * D + d] = qm[d];
          }
        }
        float amax = 0.0f;
        for (int64_t n = n0; n < n1; n++)
          for (int d = 0; d < D; d++) {
            float x = fabsf(bf16_to_f32(q[((b * Nq + n) * H + h) * D + d]) - qm[d]);
            if (x > amax) amax = x;
          }
        float s = amax / qk_max(fmt);
        q_scale[bh * nbq + t] = s;
        for (int64_t n = n0; n < n1; n++)
          for (int d = 0; d < D; d++)
            q8[(bh * Nq + n) * D + d] =
                qk_code(bf16_to_f32(q[((b * Nq + n) * H + h) * D + d]) - qm[d], s, fmt);
      }
      /* --- K mean --- */
      float mean[D];
      for (int d = 0; d < D; d++) {
        float tot = 0.0f;
        for (int64_t t = 0; t < nbk; t++) {
          int64_t n0 = t * BLK, n1 = n0 + BLK < Nkv ? n0 + BLK : Nkv;
          float part = 0.0f;
          for (int64_t n = n0; n < n1; n++) part = part + bf16_to_f32(k[((b * Nkv + n) * H + h) * D + d]);
          tot = tot + part;
        }
        mean[d] = tot / (float)Nkv;
        k_mean[bh * D + d] = mean[d];
      }
      /* --- K' codes --- */
      for (int64_t t = 0; t < nbk; t++) {
        int64_t n0 = t * BLK, n1 = n0 + BLK < Nkv ? n0 + BLK : Nkv;
        float amax = 0.0f;
        for (int64_t n = n0; n < n1; n++)
          for (int d = 0; d < D; d++) {
            float x = fabsf(bf16_to_f32(k[((b * Nkv + n) * H + h) * D + d]) - mean[d]);
            if (x > amax) amax = x;
          }
        float s = amax / qk_max(fmt);
        k_scale[bh * nbk + t] = s;
        for (int64_t n = n0; n < n1; n++)
          for (int d = 0; d < D; d++) {
            float x = bf16_to_f32(k[((b * Nkv + n) * H + h) * D + d]) - mean[d];
            k8[(bh * Nkv + n) * D + d] = qk_code(x, s, fmt);
          }
      }
      /* --- V --- */
      for (int d = 0; d < D; d++) {
        float amax = 0.0f;
        for (int64_t n = 0; n < Nkv; n++) {
          float x = fabsf(bf16_to_f32(v[((b * Nkv + n) * H + h) * D + d]));
          if (x > amax) amax = x;
        }
        float s = amax / 448.0f;
        v_scale[bh * D + d] = s;
        for (int64_t n = 0; n < Nkv; n++)
          v8[(bh * Nkv + n) * D + d] = e4m3_code(bf16_to_f32(v[((b * Nkv + n) * H + h) * D + d]), s);
      }
    }
  }
}

/* ----------------------------------------------------------- attention ---- */

/*
 * One output row (b, h, i) from the canonical codes and scales:
 *   acc_j = sum_d q8[i,d] k8[j,d]                       (exact: int32, or
 *                                                        FP64 of decoded
 *                                                        E4M3 for FP8 Q/K)
 *   s_j   = acc_j * qs * ks_blk(j) * softmax_scale      (FP64)
 *   m     = max_j s_j                                   (pass 1)
 *   p_j   = (float) exp(s_j - m)                        (pass 2; p in (0,1])
 *   l     = sum_j (double) p_j                          (key order)
 *   P8_j  = E4M3(fl32(448 * p_j))
 *   num_d = sum_j dec(P8_j) dec(V8[j,d])                (exact in FP64)
 *   o_d   = bf16(float(num_d * vs_d / (448 * l)))
 *   lse   = m + ln(l) + softmax_scale * qs * sum_d qc_d * kmean_d   (FP64)
 * With Q smoothing (`qm`, the row's block mean, non-NULL) the score gains
 * the Delta-S term that restores the block mean,
 *   s_j  += qm . kc_j * ks_blk(j) * softmax_scale         (FP64; kc: the K
 *                                                        code, decoded)
 * and the lse shift becomes softmax_scale * (qs * qc + qm) . kmean.
 * lse is the log-sum-exp of the logits before K smoothing: the scores above
 * use K - mean, and the last term adds back what that shift took from every
 * logit of the row (qc_d: the Q code, decoded for FP8).  `p` is caller
 * scratch of Nkv floats; `km` (the K mean of this (b, h)) and `lse_out` may
 * be NULL when lse is not wanted.
 * `kmask` (block-sparse attention): NULL, or the row's allowed-key-block
 * flags [nbk]; keys of other blocks take no part in m, l or the output.  A
 * row with no allowed key gets output 0 and lse = -inf.
 */
static void attention_row(const int8_t* q8, const int8_t* k8, const uint8_t* v8,
                          const float* q_scale, const float* k_scale, const float* v_scale,
                          int64_t H, int64_t Nq, int64_t Nkv, int fmt, float softmax_scale,
                          int64_t b, int64_t h, int64_t i, const float* km, const float* qm,
                          const uint8_t* kmask,
                          double* sc, float* p, uint16_t* out_row, double* m_out, double* l_out,
                          double* lse_out) {
  const int64_t bh = b * H + h;
  const int64_t nbq = nblocks(Nq), nbk = nblocks(Nkv);
  const int8_t* qi = q8 + (bh * Nq + i) * D;
  const double qs = (double)q_scale[bh * nbq + i / BLK];
  double m = -INFINITY;
  for (int64_t j = 0; j < Nkv; j++) {
    if (kmask && !kmask[j / BLK]) {
      sc[j] = -INFINITY;
      continue;
    }
    const int8_t* kj = k8 + (bh * Nkv + j) * D;
    double acc = 0.0;
    if (fmt == ORC_QK_FP8) {
      /* exact in FP64: each product is a multiple of 2^-18 below 2^18 */
      for (int d = 0; d < D; d++)
        acc += orc_e4m3_decode((uint8_t)qi[d]) * orc_e4m3_decode((uint8_t)kj[d]);
    } else {
      int32_t ia = 0;
      for (int d = 0; d < D; d++) ia += (int32_t)qi[d] * (int32_t)kj[d];
      acc = (double)ia;
    }
    if (qm) {
      double ds = 0.0;
      for (int d = 0; d < D; d++) {
        const double kc = fmt == ORC_QK_FP8 ? orc_e4m3_decode((uint8_t)kj[d]) : (double)kj[d];
        ds += (double)qm[d] * kc;
      }
      acc = acc * qs + ds;  /* in units of the K scale */
    } else {
      acc = acc * qs;
    }
    double s = acc * (double)k_scale[bh * nbk + j / BLK] * (double)softmax_scale;
    sc[j] = s;
    if (s > m) m = s;
  }
  if (m == -INFINITY) { /* no allowed key */
    for (int d = 0; d < D; d++) out_row[d] = 0;
    if (m_out) *m_out = m;
    if (l_out) *l_out = 0.0;
    if (lse_out) *lse_out = -INFINITY;
    return;
  }
  double l = 0.0;
  for (int64_t j = 0; j < Nkv; j++) {
    p[j] = (float)exp(sc[j] - m);
    l += (double)p[j];
  }
  double num[D];
  for (int d = 0; d < D; d++) num[d] = 0.0;
  for (int64_t j = 0; j < Nkv; j++) {
    double pj = orc_e4m3_decode(orc_e4m3_encode(448.0f * p[j]));
    if (pj == 0.0) continue;
    const uint8_t* vj = v8 + (bh * Nkv + j) * D;
    for (int d = 0; d < D; d++) num[d] += pj * orc_e4m3_decode(vj[d]);
  }
  for (int d = 0; d < D; d++) {
    double o = num[d] * (double)v_scale[bh * D + d] / (448.0 * l);
    out_row[d] = orc_f32_to_bf16((float)o);
  }
  if (m_out) *m_out = m;
  if (l_out) *l_out = l;
  if (lse_out) {
    double shift = 0.0;
    for (int d = 0; d < D; d++) {
      const double qc = fmt == ORC_QK_FP8 ? orc_e4m3_decode((uint8_t)qi[d]) : (double)qi[d];
      shift += (qc * qs + (qm ? (double)qm[d] : 0.0)) * (double)km[d];
    }
    *lse_out = m + log(l) + (double)softmax_scale * shift;
  }
}

/* Selected rows: rows[3r..3r+2] = (b, h, i).  out: [nrows][128] BF16;
 * m_out, l_out, lse_out: [nrows] or NULL (lse_out needs k_mean);
 * block_mask: NULL (dense) or as in orc_attention_sparse; q_mean: NULL, or
 * the Q block means [B][H][nbq][128] of a Q-smoothed quantization. */
void orc_attention_rows(const int8_t* q8, const int8_t* k8, const uint8_t* v8,
                        const float* q_scale, const float* k_scale, const float* v_scale,
                        int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int fmt, float softmax_scale,
                        int64_t nrows, const int64_t* rows, const float* k_mean,
                        const float* q_mean, const uint8_t* block_mask,
                        uint16_t* out, double* m_out, double* l_out, double* lse_out) {
  (void)B;
  const int64_t nbq = nblocks(Nq), nbk = nblocks(Nkv);
  #pragma omp parallel
  {
    double* sc = (double*)malloc(sizeof(double) * (size_t)Nkv);
    float* p = (float*)malloc(sizeof(float) * (size_t)Nkv);
    #pragma omp for schedule(dynamic)
    for (int64_t r = 0; r < nrows; r++) {
      const int64_t bh = rows[3 * r] * H + rows[3 * r + 1];
      attention_row(q8, k8, v8, q_scale, k_scale, v_scale, H, Nq, Nkv, fmt, softmax_scale,
                    rows[3 * r], rows[3 * r + 1], rows[3 * r + 2],
                    k_mean ? k_mean + bh * D : NULL,
                    q_mean ? q_mean + (bh * nbq + rows[3 * r + 2] / BLK) * D : NULL,
                    block_mask ? block_mask + (bh * nbq + rows[3 * r + 2] / BLK) * nbk : NULL,
                    sc, p, out + r * D,
                    m_out ? m_out + r : NULL, l_out ? l_out + r : NULL,
                    lse_out ? lse_out + r : NULL);
    }
    free(sc);
    free(p);
  }
}

/* Every row; out is BSHD [B][Nq][H][128] BF16; lse [B][H][Nq] or NULL
 * (then k_mean may be NULL too); q_mean as in orc_attention_rows. */
void orc_attention(const int8_t* q8, const int8_t* k8, const uint8_t* v8,
                   const float* q_scale, const float* k_scale, const float* v_scale,
                   const float* k_mean, const float* q_mean,
                   int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int fmt, float softmax_scale,
                   uint16_t* out, double* lse) {
  const int64_t nbq = nblocks(Nq);
  #pragma omp parallel
  {
    double* sc = (double*)malloc(sizeof(double) * (size_t)Nkv);
    float* p = (float*)malloc(sizeof(float) * (size_t)Nkv);
    #pragma omp for collapse(3) schedule(dynamic)
    for (int64_t b = 0; b < B; b++)
      for (int64_t h = 0; h < H; h++)
        for (int64_t i = 0; i < Nq; i++)
          attention_row(q8, k8, v8, q_scale, k_scale, v_scale, H, Nq, Nkv, fmt, softmax_scale,
                        b, h, i, lse ? k_mean + (b * H + h) * D : NULL,
                        q_mean ? q_mean + ((b * H + h) * nbq + i / BLK) * D : NULL, NULL, sc, p,
                        out + ((b * Nq + i) * H + h) * D, NULL, NULL,
                        lse ? lse + (b * H + h) * Nq + i : NULL);
    free(sc);
    free(p);
  }
}

/*
 * Block-sparse attention: query i attends key j iff
 * block_mask[b][h][i / 128][j / 128] != 0 (mask [B][H][nbq][nbk] uint8).
 * Every row as in orc_attention over its allowed keys; rows without one get
 * output 0 and lse -inf.  lse and k_mean may be NULL together; q_mean as in
 * orc_attention_rows.
 */
void orc_attention_sparse(const int8_t* q8, const int8_t* k8, const uint8_t* v8,
                          const float* q_scale, const float* k_scale, const float* v_scale,
                          const float* k_mean, const float* q_mean, const uint8_t* block_mask,
                          int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int fmt, float softmax_scale,
                          uint16_t* out, double* lse) {
  const int64_t nbq = nblocks(Nq), nbk = nblocks(Nkv);
  #pragma omp parallel
  {
    double* sc = (double*)malloc(sizeof(double) * (size_t)Nkv);
    float* p = (float*)malloc(sizeof(float) * (size_t)Nkv);
    #pragma omp for collapse(3) schedule(dynamic)
    for (int64_t b = 0; b < B; b++)
      for (int64_t h = 0; h < H; h++)
        for (int64_t i = 0; i < Nq; i++)
          attention_row(q8, k8, v8, q_scale, k_scale, v_scale, H, Nq, Nkv, fmt, softmax_scale,
                        b, h, i, lse ? k_mean + (b * H + h) * D : NULL,
                        q_mean ? q_mean + ((b * H + h) * nbq + i / BLK) * D : NULL,
                        block_mask + ((b * H + h) * nbq + i / BLK) * nbk, sc, p,
                        out + ((b * Nq + i) * H + h) * D, NULL, NULL,
                        lse ? lse + (b * H + h) * Nq + i : NULL);
    free(sc);
    free(p);
  }
}

/* ------------------------------------------------------------ exact ------ */

/* softmax(Q K^T * scale) V in FP64 from the BF16 inputs; out BSHD doubles. */
void orc_bruteforce(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                    int64_t B, int64_t H, int64_t Nq, int64_t Nkv, double softmax_scale,
                    double* out) {
  #pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)Nkv);
    #pragma omp for collapse(3) schedule(dynamic)
    for (int64_t b = 0; b < B; b++)
      for (int64_t h = 0; h < H; h++)
        for (int64_t i = 0; i < Nq; i++) {
          double m = -INFINITY;
          for (int64_t j = 0; j < Nkv; j++) {
            double acc = 0.0;
            for (int d = 0; d < D; d++)
              acc += (double)bf16_to_f32(q[((b * Nq + i) * H + h) * D + d]) *
                     (double)bf16_to_f32(k[((b * Nkv + j) * H + h) * D + d]);
            s[j] = acc * softmax_scale;
            if (s[j] > m) m = s[j];
          }
          double l = 0.0;
          for (int64_t j = 0; j < Nkv; j++) { s[j] = exp(s[j] - m); l += s[j]; }
          for (int d = 0; d < D; d++) {
            double o = 0.0;
            for (int64_t j = 0; j < Nkv; j++) o += s[j] * (double)bf16_to_f32(v[((b * Nkv + j) * H + h) * D + d]);
            out[((b * Nq + i) * H + h) * D + d] = o / l;
          }
        }
    free(s);
  }
}

int orc_rounding_mode_is_nearest(void) { return fegetround() == FE_TONEAREST; }

/* Threads an OpenMP parallel region of this library uses. */
int orc_num_threads(void) {
  int n = 1;
  #pragma omp parallel
  {
    #pragma omp single
    n = omp_get_num_threads();
  }
  return n;
}
