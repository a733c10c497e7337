// quant.hip -- preprocessing kernels: BF16 Q/K/V -> INT8 / OCP E4M3 codes.
//
// The MHA v4 page ("new MHA v4 entrypoint ...", Technical Details) keeps Q/K/V
// preprocessing apart from the attention kernel and its import listing names
// a two-stage per-channel V amax (partial kernel, finalize kernel, quantize
// kernel).  Here the same three stages serve both K and V:
//   1. stats:    per (b, h, 128-token block, channel) the FP32 sum of K over
//                the block's tokens in token order, and the max |V|.
//   2. finalize: per (b, h, channel) the K mean (block sums added in block
//                order, one division by Nkv) and the V scale amax/448.
//   3. codes:    per (b, h, block) Q and mean-smoothed K to INT8 with scale
//                amax/127 and round-half-even (or, in the FP8 Q/K format of
//                the MHA v4 page's FP8/FP8/BF16 row, to E4M3 with scale
//                amax/448); V to E4M3 with its channel scale, written
//                transposed in the attention kernel's order.
//
// The codes must equal those of the plain definition bit for bit, where the
// quotient x / s is one correctly rounded FP32 division.  A full division
// costs about ten VALU operations, more than an HBM-bound kernel can spend
// per element, so the kernels form y = x * fl(1/s) (within 2^-23 relative of
// x / s) and fall back to the exact division only when y lies so close to a
// rounding boundary that the two could round differently.  Build with
// -ffp-contract=off.
//
// With Q smoothing (the MHA v4 page's import listing: a Q-smoothing kernel
// and a Delta-S kernel) two more steps run: the Q block means (before the
// codes, which then quantize q - mean) and the Delta-S table (after them).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "kernels.h"
#include "layout.h"

namespace sattn {
namespace {

constexpr float kFltMin = 1.17549435e-38f;  // 2^-126
constexpr int64_t kStatsBlkBelow = 2 * 256 * 16;  // (b, block, head) triples: 2 k_stats workgroups per CU

__device__ inline float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ inline void unpack8(const uint4& u, float f[8]) {
  f[0] = lo_bf16(u.x); f[1] = hi_bf16(u.x);
  f[2] = lo_bf16(u.y); f[3] = hi_bf16(u.y);
  f[4] = lo_bf16(u.z); f[5] = hi_bf16(u.z);
  f[6] = lo_bf16(u.w); f[7] = hi_bf16(u.w);
}

// ------------------------------------------------------------- 1. stats ----
// One thread per (b, block t, head, 8-channel group): consecutive threads
// read consecutive 16-byte pieces of one token row, so a wave reads 1 KiB
// contiguous per token of a contiguous BSHD tensor.
struct StatsP {
  const uint16_t* k;
  const uint16_t* v;
  int64_t ks0, ks1, ks2, vs0, vs1, vs2;
  int64_t B, H, Nkv, nbk;
  float* kpart;
  float* vpart;
};

__global__ __launch_bounds__(256) void k_stats(StatsP p) {
  const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = p.B * p.nbk * p.H * 16;
  if (tid >= total) return;
  const int g = (int)(tid & 15);
  int64_t r = tid >> 4;
  const int64_t h = r % p.H;
  r /= p.H;
  const int64_t t = r % p.nbk;
  const int64_t b = r / p.nbk;
  const int64_t n0 = t * kBlk;
  const int64_t n1 = n0 + kBlk < p.Nkv ? n0 + kBlk : p.Nkv;
  const uint16_t* kp = p.k + b * p.ks0 + h * p.ks2 + 8 * g;
  const uint16_t* vp = p.v + b * p.vs0 + h * p.vs2 + 8 * g;
  float s[8], m[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) { s[c] = 0.0f; m[c] = 0.0f; }
  int64_t n = n0;
  // batches of 8 tokens: the loads are issued together, the adds stay in
  // token order
  for (; n + 8 <= n1; n += 8) {
    uint4 kk[8], vv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      kk[i] = *reinterpret_cast<const uint4*>(kp + (n + i) * p.ks1);
      vv[i] = *reinterpret_cast<const uint4*>(vp + (n + i) * p.vs1);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float kf[8], vf[8];
      unpack8(kk[i], kf);
      unpack8(vv[i], vf);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        s[c] = s[c] + kf[c];
        m[c] = fmaxf(m[c], fabsf(vf[c]));
      }
    }
  }
  for (; n < n1; ++n) {
    float kf[8], vf[8];
    unpack8(*reinterpret_cast<const uint4*>(kp + n * p.ks1), kf);
    unpack8(*reinterpret_cast<const uint4*>(vp + n * p.vs1), vf);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      s[c] = s[c] + kf[c];
      m[c] = fmaxf(m[c], fabsf(vf[c]));
    }
  }
  const int64_t o = ((b * p.H + h) * p.nbk + t) * kD + 8 * g;
  float4* ko = reinterpret_cast<float4*>(p.kpart + o);
  float4* vo = reinterpret_cast<float4*>(p.vpart + o);
  ko[0] = make_float4(s[0], s[1], s[2], s[3]);
  ko[1] = make_float4(s[4], s[5], s[6], s[7]);
  vo[0] = make_float4(m[0], m[1], m[2], m[3]);
  vo[1] = make_float4(m[4], m[5], m[6], m[7]);
}

// The same partials for short key sequences, where k_stats has a few
// workgroups whose threads each wait on 16 dependent rounds of loads.  One
// workgroup per (b, key block, head): every thread loads its 8 rows of K and
// V at once (16 bytes of one row per thread, 16 threads per row), the V
// maxima are reduced through LDS, and K is staged in LDS so that 128 threads,
// one per channel, can then add its rows in token order, the order k_stats
// uses.
__global__ __launch_bounds__(256) void k_stats_blk(StatsP p) {
  __shared__ __attribute__((aligned(16))) uint16_t kt[kBlk * kD];  // the K block, 32 KiB
  __shared__ float vred[16][kD];                                  // V maxima per row group
  const int64_t wg = blockIdx.x;  // (b, t, h), h fastest
  const int64_t h = wg % p.H;
  const int64_t t = (wg / p.H) % p.nbk;
  const int64_t b = wg / p.H / p.nbk;
  const int tid = threadIdx.x;
  const int g = tid & 15, rg = tid >> 4;  // channels 8g..8g+7 of rows rg + 16 i
  const int64_t n0 = t * kBlk;
  const int nv = (int)(p.Nkv - n0 < kBlk ? p.Nkv - n0 : kBlk);  // valid rows of the block
  const uint16_t* kp = p.k + b * p.ks0 + h * p.ks2 + 8 * g;
  const uint16_t* vp = p.v + b * p.vs0 + h * p.vs2 + 8 * g;
  uint4 kk[8], vv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = rg + 16 * i;
    kk[i] = vv[i] = make_uint4(0, 0, 0, 0);
    if (row < nv) {
      kk[i] = *reinterpret_cast<const uint4*>(kp + (n0 + row) * p.ks1);
      vv[i] = *reinterpret_cast<const uint4*>(vp + (n0 + row) * p.vs1);
    }
  }
  float m[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) m[c] = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = rg + 16 * i;
    if (row < nv) {
      float vf[8];
      unpack8(vv[i], vf);
#pragma unroll
      for (int c = 0; c < 8; ++c) m[c] = fmaxf(m[c], fabsf(vf[c]));
      *reinterpret_cast<uint4*>(kt + row * kD + 8 * g) = kk[i];
    }
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) vred[rg][8 * g + c] = m[c];
  __syncthreads();
  const int64_t o = ((b * p.H + h) * p.nbk + t) * kD;
  if (tid < kD) {
    // one channel per thread, its rows in token order
    float s = 0.0f;
#pragma unroll 16
    for (int n = 0; n < nv; ++n) s = s + __uint_as_float((uint32_t)kt[n * kD + tid] << 16);
    p.kpart[o + tid] = s;
  } else {
    const int c = tid - kD;
    float mm = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) mm = fmaxf(mm, vred[r][c]);
    p.vpart[o + c] = mm;
  }
}

// Q smoothing: per (b, Q block t, head, 8-channel group) the FP32 sum of the
// block's tokens in token order, divided once by the token count.
struct QStatsP {
  const uint16_t* q;
  int64_t qs0, qs1, qs2;
  int64_t B, H, Nq, nbq;
  float* q_mean;
};

__global__ __launch_bounds__(256) void k_qstats(QStatsP p) {
  const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (tid >= p.B * p.nbq * p.H * 16) return;
  const int g = (int)(tid & 15);
  int64_t r = tid >> 4;
  const int64_t h = r % p.H;
  r /= p.H;
  const int64_t t = r % p.nbq;
  const int64_t b = r / p.nbq;
  const int64_t n0 = t * kBlk;
  const int64_t n1 = n0 + kBlk < p.Nq ? n0 + kBlk : p.Nq;
  const uint16_t* qp = p.q + b * p.qs0 + h * p.qs2 + 8 * g;
  float s[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) s[c] = 0.0f;
  int64_t n = n0;
  for (; n + 8 <= n1; n += 8) {
    uint4 qq[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) qq[i] = *reinterpret_cast<const uint4*>(qp + (n + i) * p.qs1);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float qf[8];
      unpack8(qq[i], qf);
#pragma unroll
      for (int c = 0; c < 8; ++c) s[c] = s[c] + qf[c];
    }
  }
  for (; n < n1; ++n) {
    float qf[8];
    unpack8(*reinterpret_cast<const uint4*>(qp + n * p.qs1), qf);
#pragma unroll
    for (int c = 0; c < 8; ++c) s[c] = s[c] + qf[c];
  }
  const float cnt = (float)(n1 - n0);
  float* o = p.q_mean + ((b * p.H + h) * p.nbq + t) * kD + 8 * g;
  reinterpret_cast<float4*>(o)[0] = make_float4(__fdiv_rn(s[0], cnt), __fdiv_rn(s[1], cnt),
                                                __fdiv_rn(s[2], cnt), __fdiv_rn(s[3], cnt));
  reinterpret_cast<float4*>(o)[1] = make_float4(__fdiv_rn(s[4], cnt), __fdiv_rn(s[5], cnt),
                                                __fdiv_rn(s[6], cnt), __fdiv_rn(s[7], cnt));
}

// ---------------------------------------------------------- 2. finalize ----
struct FinP {
  const float* kpart;
  const float* vpart;
  int64_t BH, nbk, Nkv;
  float* k_mean;
  float* v_scale;
};

// One workgroup per (b, h, 32-channel group).  The block partials are staged
// through LDS 64 blocks at a time (the next chunk's loads are in flight while
// the current one is summed), so the serial FP32 sum over blocks waits on LDS,
// not on one HBM round trip per block.
constexpr int kFinChunk = 64;

__global__ __launch_bounds__(256) void k_finalize(FinP p) {
  __shared__ float sk[kFinChunk][32];
  __shared__ float sv[kFinChunk][32];
  const int64_t bh = blockIdx.x;
  const int c0 = 32 * (int)blockIdx.y;
  const int tid = threadIdx.x;
  const float* kp = p.kpart + bh * p.nbk * kD + c0;
  const float* vp = p.vpart + bh * p.nbk * kD + c0;
  float4 rk[2], rv[2];
  auto fetch = [&](int64_t t0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + 256 * i;
      const int64_t t = t0 + (idx >> 3);
      const int c = 4 * (idx & 7);
      rk[i] = rv[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if (t < p.nbk) {
        rk[i] = *reinterpret_cast<const float4*>(kp + t * kD + c);
        rv[i] = *reinterpret_cast<const float4*>(vp + t * kD + c);
      }
    }
  };
  float tot = 0.0f, m = 0.0f;
  fetch(0);
  for (int64_t t0 = 0; t0 < p.nbk; t0 += kFinChunk) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + 256 * i;
      *reinterpret_cast<float4*>(&sk[idx >> 3][4 * (idx & 7)]) = rk[i];
      *reinterpret_cast<float4*>(&sv[idx >> 3][4 * (idx & 7)]) = rv[i];
    }
    __syncthreads();
    fetch(t0 + kFinChunk);
    const int cnt = (int)(p.nbk - t0 < kFinChunk ? p.nbk - t0 : kFinChunk);
    if (tid < 32) {
      for (int t = 0; t < cnt; ++t) tot = tot + sk[t][tid];
    } else if (tid < 64) {
      for (int t = 0; t < cnt; ++t) m = fmaxf(m, sv[t][tid - 32]);
    }
    __syncthreads();
  }
  if (tid < 32) p.k_mean[bh * kD + c0 + tid] = __fdiv_rn(tot, (float)p.Nkv);
  else if (tid < 64) p.v_scale[bh * kD + c0 + tid - 32] = __fdiv_rn(m, 448.0f);
}

// ------------------------------------------------------------- 3. codes ----

// clamp(RNE(x / s), -127, 127), s > 0.  `r` = fl(1/s), `exact` when s is
// subnormal (then fl(1/s) may overflow and x*r is no longer within 2^-23).
__device__ inline int int8_code(float x, float s, float r, bool exact) {
  float y = exact ? __fdiv_rn(x, s) : x * r;
  float t = __builtin_rintf(y);
  // |y - x/s| <= 2^-16 for |x/s| <= 128, and fl(x/s) is within 2^-17 of
  // x/s: unless y is within 2^-15 of a half-integer both round alike.
  if (!exact && fabsf(y - t) > 0.499969482421875f) t = __builtin_rintf(__fdiv_rn(x, s));
  t = fminf(fmaxf(t, -127.0f), 127.0f);
  return (int)t;
}

__device__ inline float clamp448(float y) { return fminf(fmaxf(y, -448.0f), 448.0f); }

// Hardware FP32 -> OCP E4M3, round to nearest even, for |y| <= 448.
__device__ inline uint32_t e4m3_hw(float y) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y, 0.0f, 0, false) & 0xFFu;
}

// E4M3(clamp(v / s, +-448)), s > 0.  The exact quotient lies between
// y(1 - 2^-20) and y(1 + 2^-20); rounding is monotone, so when both ends give
// the same code that code is the answer.
__device__ inline uint32_t e4m3_code(float v, float s, float r, bool exact) {
  if (exact) return e4m3_hw(clamp448(__fdiv_rn(v, s)));
  const float y = v * r;
  const uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
      clamp448(y * 0.99999904632568359375f), clamp448(y * 1.00000095367431640625f), 0, false);
  if ((w & 0xFFu) == ((w >> 8) & 0xFFu)) return w & 0xFFu;
  return e4m3_hw(clamp448(__fdiv_rn(v, s)));
}

// x from another lane under a DPP control (all rows and banks enabled)
template <int CTRL>
__device__ inline float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Maximum over the wave, in every lane, without LDS: DPP within each row of
// 16 lanes (quad permutations, then rotations by 4 and 8), then the row
// swaps of gfx950 (v_permlane16_swap, v_permlane32_swap) across rows.
// A maximum is exact, so the order does not change the result.
__device__ inline float wave_max(float a) {
  a = fmaxf(a, dpp_f<0xB1>(a));   // quad_perm [1, 0, 3, 2]
  a = fmaxf(a, dpp_f<0x4E>(a));   // quad_perm [2, 3, 0, 1]
  a = fmaxf(a, dpp_f<0x124>(a));  // row_ror:4
  a = fmaxf(a, dpp_f<0x128>(a));  // row_ror:8
  const int x = __float_as_int(a);
  const auto r16 = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  a = fmaxf(__int_as_float((int)r16[0]), __int_as_float((int)r16[1]));
  const int y = __float_as_int(a);
  const auto r32 = __builtin_amdgcn_permlane32_swap(y, y, false, false);
  return fmaxf(__int_as_float((int)r32[0]), __int_as_float((int)r32[1]));
}

struct CodeP {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  int64_t qs0, qs1, qs2, ks0, ks1, ks2, vs0, vs1, vs2;
  int64_t H, Nq, Nkv, nbq, nbk, BH;
  int fp8qk;
  uint8_t* q8;
  uint8_t* k8;
  uint8_t* v8;
  float* q_scale;
  float* k_scale;
  const float* v_scale;
  const float* k_mean;
  const float* q_mean;  // Q smoothing: block means [BH][nbq][128], or null
};

// One workgroup of 256 threads per (tensor, b, h, 128-token block).  Thread
// (tg, cg) holds tokens 8tg..8tg+7 x channels 8cg..8cg+7 of the block.
__global__ __launch_bounds__(256) void k_codes(CodeP p) {
  __shared__ __attribute__((aligned(16))) uint8_t vt[kTileBytes];
  __shared__ float red[4];
  const int64_t wid = blockIdx.x;
  const int tid = threadIdx.x;
  const int tg = tid >> 4, cg = tid & 15;
  int kind;  // 0 = Q, 1 = K, 2 = V
  int64_t b, h, t;
  const int64_t nkv = p.BH * p.nbk;
  if (wid < 2 * nkv) {
    // K and V blocks first, alternating, in the reverse of the order the
    // stats step read them ((b, t, h) ascending): the blocks it read last
    // are the likeliest to still sit in the memory-side cache.
    kind = 1 + (int)(wid & 1);
    int64_t r = nkv - 1 - (wid >> 1);
    h = r % p.H;
    r /= p.H;
    t = r % p.nbk;
    b = r / p.nbk;
  } else {
    kind = 0;
    const int64_t u = wid - 2 * nkv;
    const int64_t bq = u / p.nbq;
    t = u % p.nbq;
    b = bq / p.H;
    h = bq % p.H;
  }
  const int64_t bh = b * p.H + h;
  const int64_t N = kind == 0 ? p.Nq : p.Nkv;
  const uint16_t* src;
  int64_t s0, s1, s2;
  if (kind == 0) { src = p.q; s0 = p.qs0; s1 = p.qs1; s2 = p.qs2; }
  else if (kind == 1) { src = p.k; s0 = p.ks0; s1 = p.ks1; s2 = p.ks2; }
  else { src = p.v; s0 = p.vs0; s1 = p.vs1; s2 = p.vs2; }
  const uint16_t* base = src + b * s0 + h * s2 + 8 * cg;
  const int64_t n_base = t * kBlk + 8 * tg;

  float x[8][8];
  bool valid[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    valid[i] = n_base + i < N;
    uint4 u = make_uint4(0, 0, 0, 0);
    if (valid[i]) u = *reinterpret_cast<const uint4*>(base + (n_base + i) * s1);
    unpack8(u, x[i]);
  }

  if (kind == 2) {
    // ---- V: channel scales from the finalize step; E4M3 codes written into
    // an LDS copy of the V^T tile, then copied out in 16-byte pieces.
    float sc[8], rc[8];
    bool ex[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      sc[c] = p.v_scale[bh * kD + 8 * cg + c];
      ex[c] = sc[c] < kFltMin;
      rc[c] = ex[c] ? 0.0f : __fdiv_rn(1.0f, sc[c]);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      uint32_t w0 = 0, w1 = 0;
      if (sc[c] != 0.0f) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          uint32_t code = valid[i] ? e4m3_code(x[i][c], sc[c], rc[c], ex[c]) : 0u;
          if (i < 4) w0 |= code << (8 * i);
          else w1 |= code << (8 * (i - 4));
        }
      }
      const int d = 8 * cg + c;
      const int key = 8 * tg;
      *reinterpret_cast<uint32_t*>(vt + v_pos(key, d)) = w0;
      *reinterpret_cast<uint32_t*>(vt + v_pos(key + 4, d)) = w1;
    }
    __syncthreads();
    uint4* dst = reinterpret_cast<uint4*>(p.v8 + (bh * p.nbk + t) * kTileBytes);
    const uint4* s = reinterpret_cast<const uint4*>(vt);
#pragma unroll
    for (int j = 0; j < 4; ++j) dst[tid + 256 * j] = s[tid + 256 * j];
    return;
  }

  // ---- Q and K: block amax, scale amax/127 with INT8 codes, or amax/448
  // with E4M3 codes (the FP8 Q/K format).
  // K: subtract the sequence mean; Q with smoothing: the block mean
  const float* mrow = kind == 1 ? p.k_mean + bh * kD
                    : p.q_mean != nullptr ? p.q_mean + (bh * p.nbq + t) * kD : nullptr;
  if (mrow != nullptr) {
    float mean[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) mean[c] = mrow[8 * cg + c];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int c = 0; c < 8; ++c) x[i][c] = valid[i] ? x[i][c] - mean[c] : 0.0f;
  }
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int c = 0; c < 8; ++c)
      if (valid[i]) am = fmaxf(am, fabsf(x[i][c]));
  am = wave_max(am);
  if ((tid & 63) == 0) red[tid >> 6] = am;
  __syncthreads();
  am = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = __fdiv_rn(am, p.fp8qk ? 448.0f : 127.0f);
  const bool ex = s < kFltMin;
  const float r = ex ? 0.0f : __fdiv_rn(1.0f, s);
  if (tid == 0) (kind == 0 ? p.q_scale : p.k_scale)[bh * (kind == 0 ? p.nbq : p.nbk) + t] = s;
  uint8_t* tile = (kind == 0 ? p.q8 + (bh * p.nbq + t) * kTileBytes : p.k8 + (bh * p.nbk + t) * kTileBytes);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t w[2] = {0u, 0u};
    if (valid[i] && s != 0.0f) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint32_t code = p.fp8qk ? e4m3_code(x[i][c], s, r, ex) : (uint32_t)(int8_code(x[i][c], s, r, ex) & 0xFF);
        w[c >> 2] |= code << (8 * (c & 3));
      }
    }
    const int row = 8 * tg + i;
    const int pos = kind == 0 ? q_pos(row, 8 * cg) : k_pos(row, 8 * cg);
    *reinterpret_cast<uint2*>(tile + pos) = make_uint2(w[0], w[1]);
  }
}

// ------------------------------------------------------------ 4. Delta-S ----
// With INT8 codes the attention kernel forms Delta-S itself from k_qdigits'
// digit rows (after this kernel).  The E4M3 Q/K format keeps a table:
// D[bh][i][t*128 + j] = (q_mean[bh][i] . kcode(t, j)) / u_i for every Q block
// i, u_i = qs_i (2^-20 when qs_i = 0, a block of equal tokens: its scores
// are Delta-S alone, kept at FP32 resolution): the score term that restores
// the Q block mean, in the units of the Q.K^T accumulator (times qs * ks it
// is the score), so the attention kernel adds it to the accumulator as it
// is.  The codes of keys past Nkv are zero, so their entries are too.
//
// Per (b, h) this is a [nbq x 128] x [128 x Nkv] FP32 product: it runs on
// the FP32 MFMA (32x32x2), whose rate is twice that of FP32 FMAs on the
// vector ALU.  The decoded codes are exact in FP32.  One workgroup of four
// waves per (b, h, key tile); wave w holds the 32 keys 32w.. of the tile as
// the B operand (64 registers: lane half h supplies channel 64h + s at step
// s) and sweeps the Q blocks 32 at a time, the means of its 32 blocks times
// 1 / u as the A operand (lane l: block l % 32, channels 64h .. 64h + 63),
// loading the next group's means while the MFMAs of this one run.
struct DsP {
  const uint8_t* k8;
  const float* q_scale;
  const float* q_mean;
  float* ds;
  int64_t nbq, nbk;
};

typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void k_delta_s(DsP p) {
  const int64_t g = blockIdx.x;  // bh * nbk + t
  const int64_t bh = g / p.nbk, t = g % p.nbk;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = lane & 31, h = lane >> 5;
  const int key = 32 * w + col;
  // B operand: channels 64h .. 64h + 63 of this lane's key, i.e. the logical
  // 16-byte chunks 4h .. 4h + 3 of its row
  const uint8_t* row = p.k8 + g * kTileBytes + key * 128;
  float kb[64];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint4 u = *reinterpret_cast<const uint4*>(row + ((((4 * h + c) ^ swz(key)) & 7) << 4));
    const int wd[4] = {(int)u.x, (int)u.y, (int)u.z, (int)u.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      kb[16 * c + 4 * q + 0] = __builtin_amdgcn_cvt_f32_fp8(wd[q], 0);
      kb[16 * c + 4 * q + 1] = __builtin_amdgcn_cvt_f32_fp8(wd[q], 1);
      kb[16 * c + 4 * q + 2] = __builtin_amdgcn_cvt_f32_fp8(wd[q], 2);
      kb[16 * c + 4 * q + 3] = __builtin_amdgcn_cvt_f32_fp8(wd[q], 3);
    }
  }
  const float* qsr = p.q_scale + bh * p.nbq;
  const float* qm = p.q_mean + bh * p.nbq * kD;
  float* out = p.ds + bh * p.nbq * (p.nbk * kBlk) + t * kBlk + key;
  // A operand of a group of 32 Q blocks: this lane's block mean, divided by
  // that block's u (one division per lane, then a multiply per mean)
  auto load_a = [&](int64_t i0, float (&qa)[64]) __attribute__((always_inline)) {
    const int64_t ia = i0 + col;
    if (ia < p.nbq) {
      const float4* src = reinterpret_cast<const float4*>(qm + ia * kD + 64 * h);
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const float4 m4 = src[c];
        qa[4 * c] = m4.x; qa[4 * c + 1] = m4.y; qa[4 * c + 2] = m4.z; qa[4 * c + 3] = m4.w;
      }
    } else {
#pragma unroll
      for (int c = 0; c < 64; ++c) qa[c] = 0.0f;
    }
  };
  auto scale_a = [&](int64_t i0, float (&qa)[64]) __attribute__((always_inline)) {
    const int64_t ia = i0 + col;
    const float u = ia < p.nbq ? qsr[ia] : 1.0f;
    const float r = u > 0.0f ? __fdiv_rn(1.0f, u) : 0x1p20f;
#pragma unroll
    for (int c = 0; c < 64; ++c) qa[c] *= r;
  };
  float qa[64], qn[64];
  load_a(0, qa);
  for (int64_t i0 = 0; i0 < p.nbq; i0 += 32) {
    scale_a(i0, qa);
    if (i0 + 32 < p.nbq) load_a(i0 + 32, qn);  // the next group's means, in flight during the MFMAs
    f32x16 acc = {};
#pragma unroll
    for (int st = 0; st < 64; ++st) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[st], kb[st], acc, 0, 0, 0);
    // accumulator row of register r: Q block i0 + 8(r / 4) + 4h + r % 4
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t i = i0 + 8 * (r >> 2) + 4 * h + (r & 3);
      if (i < p.nbq) out[i * (p.nbk * kBlk)] = acc[r];
    }
#pragma unroll
    for (int c = 0; c < 64; ++c) qa[c] = qn[c];
  }
}

// Q smoothing with INT8 codes: the block mean in the form the attention
// kernel multiplies with the K codes on the INT8 MFMA, per (b, h, Q block):
//   unit  the block's score unit: the accumulator of Qcode . Kcode counts
//         units of unit * ks.  It is qs, times 2^k when the mean is more
//         than 2^15 units (then the kernel rounds the Q codes to multiples
//         of 2^k); for qs = 0 (equal tokens, all-zero codes) amax|mean| * 2^-14.
//   u_d = mean_d / unit, so |u_d| < 2^15 and, with |Kcode| <= 127, the
//         correction sum_d u_d Kcode_d and the code product both fit the
//         accumulator's 32 bits (< 2^29 and <= 2^21);
//   digit rows a_0..a_3 (int8, |a_r| <= 64) with
//         u_d = 2^E (a_0 + 2^-7 a_1 + 2^-14 a_2 + 2^-21 a_3) + e_d,
//         E = ilogb(max_d |u_d|) - 5, |e_d| <= 2^(E-22) (each remainder is
//         exact in FP32: it is a multiple of the ulp of u_d below 2^24 of them);
//   params  {unit, 2^E, 2^(E-7), 2^(E-14), 2^(E-21), k (int bits), 0, 0}.
// One wave per block, two channels per lane; quant.hip is built without FP
// contraction, so each step is one IEEE operation.
struct DigP {
  const float* q_scale;
  const float* q_mean;
  int8_t* dg;
  float* dp;
  int64_t nblk;
};

__global__ __launch_bounds__(256) void k_qdigits(DigP p) {
  const int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (blk >= p.nblk) return;  // wave-uniform
  const int lane = threadIdx.x & 63;
  const float2 m2 = reinterpret_cast<const float2*>(p.q_mean + blk * kD)[lane];
  const float qs = p.q_scale[blk];
  const float amax = wave_max(fmaxf(fabsf(m2.x), fabsf(m2.y)));
  int k = 0;
  float unit;
  if (qs > 0.0f) {
    // amax / (qs 2^k) < 2^(ilogb(amax) + 1 - ilogb(qs) - k) <= 2^15
    if (amax > 0.0f) k = max(0, ilogbf(amax) - ilogbf(qs) - 14);
    unit = ldexpf(qs, k);
  } else {
    unit = amax > 0.0f ? fmaxf(ldexpf(amax, -14), 1.17549435e-38f) : 1.0f;
  }
  const float u[2] = {__fdiv_rn(m2.x, unit), __fdiv_rn(m2.y, unit)};
  const float mu = wave_max(fmaxf(fabsf(u[0]), fabsf(u[1])));
  const int E = mu > 0.0f ? ilogbf(mu) - 5 : 0;
  int dig[4][2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    float r = u[c];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // the clamp only acts where the weights underflow (E near -149)
      const float a = fminf(fmaxf(rintf(ldexpf(r, 7 * j - E)), -127.0f), 127.0f);
      dig[j][c] = (int)a;
      r = r - ldexpf(a, E - 7 * j);
    }
  }
  int8_t* dst = p.dg + blk * kDigitBytes + 2 * lane;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    *reinterpret_cast<uint16_t*>(dst + 128 * j) = (uint16_t)((dig[j][0] & 0xFF) | ((dig[j][1] & 0xFF) << 8));
  if (lane < kDigitParams) {
    float v = 0.0f;
    if (lane == 0) v = unit;
    else if (lane <= 4) v = mu > 0.0f ? ldexpf(1.0f, E - 7 * (lane - 1)) : 0.0f;
    else if (lane == 5) v = __int_as_float(k);
    p.dp[blk * kDigitParams + lane] = v;
  }
}

__global__ __launch_bounds__(256) void k_e4m3(const float* x, uint8_t* out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = (uint8_t)e4m3_hw(clamp448(x[i]));
}

}  // namespace

// Workspace of sattn_quantize_qkv_noalloc, for callers that cannot allocate:
// a file-scope device array (one per GPU, held until the process ends) in
// place of the caller's workspace.  Its contents need no clearing: the
// statistics kernels write every partial before anything reads it.  Calls
// that overlap on one GPU share it and race.
static __device__ __attribute__((aligned(256))) uint8_t scratch[kNoallocWorkspaceBytes];

hipError_t noalloc_workspace(uint8_t** out) {
  constexpr int kMaxDev = 64;
  static std::atomic<uint8_t*> addr[kMaxDev];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  uint8_t* ptr = addr[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    // the array's name is a host-side stand-in: its device address comes
    // from the runtime, once per device, with that device current
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptr = static_cast<uint8_t*>(a);
    addr[dev].store(ptr, std::memory_order_release);
  }
  *out = ptr;
  return hipSuccess;
}

hipError_t launch_quantize(const QuantArgs& a, hipStream_t stream) {
  const Layout& L = a.L;
  const int64_t BH = L.B * L.H;
  float* kpart = reinterpret_cast<float*>(a.workspace + L.ws_kpart);
  float* vpart = reinterpret_cast<float*>(a.workspace + L.ws_vpart);
  float* q_scale = reinterpret_cast<float*>(a.packed + L.off_qs);
  float* k_scale = reinterpret_cast<float*>(a.packed + L.off_ks);
  float* v_scale = reinterpret_cast<float*>(a.packed + L.off_vs);
  float* k_mean = reinterpret_cast<float*>(a.packed + L.off_km);

  StatsP sp{a.k, a.v, a.k_str[0], a.k_str[1], a.k_str[2], a.v_str[0], a.v_str[1], a.v_str[2],
            L.B, L.H, L.Nkv, L.nbk, kpart, vpart};
  // k_stats runs one thread per (b, block, head, 8 channels); below two of
  // its workgroups per CU the per-block kernel is faster (same values)
  const int64_t sblocks = L.B * L.nbk * L.H;
  if (sblocks < kStatsBlkBelow) {
    hipLaunchKernelGGL(k_stats_blk, dim3((unsigned)sblocks), dim3(256), 0, stream, sp);
  } else {
    const int64_t sthreads = sblocks * 16;
    hipLaunchKernelGGL(k_stats, dim3((unsigned)((sthreads + 255) / 256)), dim3(256), 0, stream, sp);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  float* q_mean = L.qsmooth ? reinterpret_cast<float*>(a.packed + L.off_qm) : nullptr;
  if (L.qsmooth) {
    QStatsP qp{a.q, a.q_str[0], a.q_str[1], a.q_str[2], L.B, L.H, L.Nq, L.nbq, q_mean};
    const int64_t qthreads = L.B * L.nbq * L.H * 16;
    hipLaunchKernelGGL(k_qstats, dim3((unsigned)((qthreads + 255) / 256)), dim3(256), 0, stream, qp);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }

  FinP fp{kpart, vpart, BH, L.nbk, L.Nkv, k_mean, v_scale};
  hipLaunchKernelGGL(k_finalize, dim3((unsigned)BH, 4), dim3(256), 0, stream, fp);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  CodeP cp{a.q, a.k, a.v,
           a.q_str[0], a.q_str[1], a.q_str[2], a.k_str[0], a.k_str[1], a.k_str[2],
           a.v_str[0], a.v_str[1], a.v_str[2],
           L.H, L.Nq, L.Nkv, L.nbq, L.nbk, BH, a.fp8qk ? 1 : 0,
           a.packed + L.off_q8, a.packed + L.off_k8, a.packed + L.off_v8,
           q_scale, k_scale, v_scale, k_mean, q_mean};
  hipLaunchKernelGGL(k_codes, dim3((unsigned)(BH * (L.nbq + 2 * L.nbk))), dim3(256), 0, stream, cp);
  e = hipGetLastError();
  if (e != hipSuccess || !L.qsmooth) return e;
  if (!a.fp8qk) {
    DigP gp{q_scale, q_mean, reinterpret_cast<int8_t*>(a.packed + L.off_dg),
            reinterpret_cast<float*>(a.packed + L.off_dp), BH * L.nbq};
    hipLaunchKernelGGL(k_qdigits, dim3((unsigned)((BH * L.nbq + 3) / 4)), dim3(256), 0, stream, gp);
    return hipGetLastError();
  }
  DsP dp{a.packed + L.off_k8, q_scale, q_mean, reinterpret_cast<float*>(a.packed + L.off_ds), L.nbq, L.nbk};
  hipLaunchKernelGGL(k_delta_s, dim3((unsigned)(BH * L.nbk)), dim3(256), 0, stream, dp);
  return hipGetLastError();
}

hipError_t launch_e4m3_encode(const float* x, uint8_t* out, int64_t n, hipStream_t stream) {
  hipLaunchKernelGGL(k_e4m3, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, x, out, n);
  return hipGetLastError();
}

}  // namespace sattn
