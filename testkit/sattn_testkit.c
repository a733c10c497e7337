/*
 * sattn_testkit.c -- seeded, counter-based synthetic inputs for the attention
 * tests and benchmark.  It holds none of the method's arithmetic: it only
 * draws BF16 Q/K/V tensors with the value distributions of diffusion-
 * transformer attention workloads (Gaussian activations, per-channel key
 * bias, outlier channels, heavy tails).
 *
 * Random words: SplitMix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014), used as a counter-based
 * hash:  word(seed, stream, index, j) = f(f(f(seed) ^ stream) ^ (4*index + j)),
 * where f(x) = mix(x + 0x9E3779B97F4A7C15) is the SplitMix64 output function.
 * Normals: Box-Muller in FP64 (cosine branch).  Student-t with nu = 4:
 * z / sqrt(chi2_4 / 4), chi2_4 = -2 ln u3 - 2 ln u4, scaled by 1/sqrt(2) to
 * unit variance.  Each element is computed in FP64 and rounded once to BF16
 * (round to nearest even).
 *
 * Element (b, n, h, d) uses index ((b * 2^12 + h) * 2^25 + n) * 2^7 + d, so its
 * value depends on neither the memory layout nor the tensor extents: a
 * smaller tensor of the same recipe is a sub-block of a larger one.
 */
#include <stdint.h>
#include <string.h>
#include <math.h>

static uint64_t sm_mix(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static uint64_t tk_word(uint64_t seed, uint64_t stream, uint64_t index, uint64_t j) {
  return sm_mix(sm_mix(sm_mix(seed) ^ stream) ^ (4ull * index + j));
}

uint64_t tk_word_export(uint64_t seed, uint64_t stream, uint64_t index, uint64_t j) {
  return tk_word(seed, stream, index, j);
}

/* uniform in (0, 1] and in [0, 1) from the top 53 bits */
static double u_open0(uint64_t w) { return (double)((w >> 11) + 1) * 0x1.0p-53; }
static double u_open1(uint64_t w) { return (double)(w >> 11) * 0x1.0p-53; }

static double tk_normal(uint64_t seed, uint64_t stream, uint64_t idx) {
  double u1 = u_open0(tk_word(seed, stream, idx, 0));
  double u2 = u_open1(tk_word(seed, stream, idx, 1));
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}

static double tk_student4(uint64_t seed, uint64_t stream, uint64_t idx) {
  double z = tk_normal(seed, stream, idx);
  double u3 = u_open0(tk_word(seed, stream, idx, 2));
  double u4 = u_open0(tk_word(seed, stream, idx, 3));
  double chi2 = -2.0 * log(u3) - 2.0 * log(u4);
  return z / sqrt(chi2 / 4.0) * 0.7071067811865476;
}

/* FP64 -> BF16 with a single round-to-nearest-even: FP64 -> FP32 rounded to
   odd (exact for the later rounding since FP32 keeps 16 more bits), then
   FP32 -> BF16 RNE. */
static uint16_t d_to_bf16(double x) {
  float f = (float)x;
  if (fabs((double)f) > fabs(x)) f = nextafterf(f, 0.0f);
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((double)f != x) u |= 1u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

uint16_t tk_d_to_bf16(double x) { return d_to_bf16(x); }

enum { TK_NORMAL = 0, TK_STUDENT4 = 1 };

/*
 * Fill out[B][N][H][D] (BF16 bits) with  mult(h,d) * z + bias(h,d)  where z
 * has distribution `dist`, bias(h,d) ~ N(0, bias_sigma^2) drawn from stream
 * `bias_stream` (shared by every token and batch item; 0 sigma = no bias), and
 * mult(h,d) = outlier_mult on one channel per head (drawn from stream
 * `outlier_stream`, uniform over D) when outlier_mult != 1, else 1.
 */
void tk_fill(uint16_t* out, int64_t B, int64_t N, int64_t H, int64_t D,
             uint64_t seed, uint64_t stream, int dist,
             double bias_sigma, uint64_t bias_stream,
             double outlier_mult, uint64_t outlier_stream) {
  #pragma omp parallel for collapse(2) schedule(static)
  for (int64_t b = 0; b < B; b++)
    for (int64_t h = 0; h < H; h++) {
      int64_t och = -1;
      if (outlier_mult != 1.0)
        och = (int64_t)(u_open1(tk_word(seed, outlier_stream, (uint64_t)h, 0)) * (double)D);
      for (int64_t n = 0; n < N; n++)
        for (int64_t d = 0; d < D; d++) {
          uint64_t idx = ((((uint64_t)b << 12 | (uint64_t)h) << 25 | (uint64_t)n) << 7) | (uint64_t)d;
          double z = dist == TK_STUDENT4 ? tk_student4(seed, stream, idx) : tk_normal(seed, stream, idx);
          double mult = d == och ? outlier_mult : 1.0;
          double bias = 0.0;
          if (bias_sigma != 0.0) bias = bias_sigma * tk_normal(seed, bias_stream, (uint64_t)(h * D + d));
          out[((b * N + n) * H + h) * D + d] = d_to_bf16(mult * z + bias);
        }
    }
}
