// attn_fwd.hip -- INT8-QK / FP8-PV attention forward for gfx950.
//
// Operands as the gfx1201 backend page states them ("[ROCm] Add
// aiter_sage_attn attention backend for gfx1201 (RDNA4)", Changes): INT8
// Q.K^T, FP8 P.V, FP32 accumulation, head dim 128, non-causal; BF16 output as
// in the INT8/FP8/BF16 row of the MI355X table of the MHA v4 page.  The MHA v4
// page (Motivation) names the levers this kernel is built around: the
// softmax rescale is conditional (skipped for a wave when no row maximum of
// the tile grew), the exponentials run on the VALU in base 2 (log2(e) folded
// into the dequantisation scale), and MFMA, VALU and loads are overlapped
// (two LDS stages: the next K/V tile is fetched while the current one is
// consumed).
//
// Data flow per wave (QB blocks of 32 queries; 128-key tiles):
//   S^T = K8 . Q8^T   v_mfma_i32_32x32x32_i8, A = K tile rows from LDS,
//                     B = the wave's Q codes held in VGPRs for the whole
//                     kernel.  The accumulator leaves each lane one query
//                     (lane % 32) and 16 keys per 32-key block, so the row
//                     max and row sum are lane-local plus one exchange with
//                     the other lane half.
//   softmax           t = float(acc) * c with c = qs * ks * scale * log2(e);
//                     the tile max is taken on the integers (c > 0 is uniform
//                     over the tile); p448 = exp2(t - m + log2 448).
//   P8                v_cvt_pk_fp8_f32 packs four p values per VGPR; the V^T
//                     tile columns were permuted by the quantizer so these
//                     registers are already the B operand of the PV MFMA.
//   O^T += V8^T . P8  v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales;
//                     each lane again holds one query, so the rescale by
//                     alpha = exp2(m_old - m_new) is a per-lane multiply.
//   epilogue          O = acc * vs[d] / l448, BF16 round-to-nearest-even.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kernels.h"
#include "layout.h"

namespace sattn {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLog2_448 = 8.80735492205760410744f;
constexpr int kStageBytes = 2 * (int)kTileBytes;  // K tile + V^T tile

struct AttnP {
  const uint8_t* q8;
  const uint8_t* k8;
  const uint8_t* v8;
  const float* qs;
  const float* ks;
  const float* vs;
  uint16_t* out;
  int64_t os0, os1, os2;
  int64_t G;   // logical workgroups: B*H*mt
  int H, Nq, Nkv, nbq, nbk, mt;
  float sl2e;  // softmax_scale * log2(e)
};

__device__ inline int other_half_i(int x) {
  // lanes l and l^32 exchange x; both results hold {x_l, x_l^32}
  auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return (threadIdx.x & 32) ? (int)r[0] : (int)r[1];
}
__device__ inline float other_half_f(float x) { return __int_as_float(other_half_i(__float_as_int(x))); }

__device__ inline uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <int QB, int NW>
__global__ __launch_bounds__(NW * 64) void attn_fwd_kernel(AttnP p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr int NT = NW * 64;
  constexpr int BM = NW * QB * 32;
  constexpr int NCH = 2 * (int)kTileBytes / 16 / NT;  // 16-byte pieces per thread per stage
  static_assert(NCH * NT * 16 == kStageBytes, "stage must split evenly");
  static_assert((1024 % NT) == 0, "K/V halves must split evenly");

  // Workgroups are dispatched round-robin over the 8 XCDs; remap so that the
  // workgroups resident on one XCD take consecutive q-tiles of the same head
  // and share its K/V tiles in that XCD's L2.
  const int64_t G8 = (p.G + 7) / 8 * 8;
  const int64_t wg = blockIdx.x;
  const int64_t L = (wg % 8) * (G8 / 8) + wg / 8;
  if (L >= p.G) return;
  const int64_t bh = L / p.mt;
  const int mtile = (int)(L % p.mt);
  const int64_t b = bh / p.H, h = bh % p.H;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int q0 = mtile * BM + w * QB * 32;  // first query of this wave
  const int qblk = q0 >> 7;

  // ---- the wave's Q codes (B operand of S^T), resident for the whole loop
  v4i qf[QB][4];
  float qscale = 0.0f;
  if (q0 < p.nbq * 128) {
    const uint8_t* qt = p.q8 + (bh * p.nbq + qblk) * kTileBytes;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const v4i* src = reinterpret_cast<const v4i*>(qt + ((q0 & 127) + 32 * qb + l32) * 128 + 64 * hh);
#pragma unroll
      for (int m = 0; m < 4; ++m) qf[qb][m] = src[m];
    }
    qscale = p.qs[bh * p.nbq + qblk];
  } else {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int m = 0; m < 4; ++m) qf[qb][m] = v4i{0, 0, 0, 0};
  }

  const uint8_t* kbase = p.k8 + bh * p.nbk * kTileBytes;
  const uint8_t* vbase = p.v8 + bh * p.nbk * kTileBytes;
  const float* ksc = p.ks + bh * p.nbk;

  v4i stg[NCH];
  auto gload = [&](int t) {
    const v4i* kt = reinterpret_cast<const v4i*>(kbase + (int64_t)t * kTileBytes);
    const v4i* vt = reinterpret_cast<const v4i*>(vbase + (int64_t)t * kTileBytes);
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int c = tid + j * NT;
      stg[j] = c < 1024 ? kt[c] : vt[c - 1024];
    }
  };
  auto swrite = [&](int s) {
    v4i* dst = reinterpret_cast<v4i*>(smem + s * kStageBytes);
#pragma unroll
    for (int j = 0; j < NCH; ++j) dst[tid + j * NT] = stg[j];
  };

  float m_run[QB], l_run[QB];
  v16f O[4][QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -__builtin_inff();
    l_run[qb] = 0.0f;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) O[db][qb][r] = 0.0f;
  }

  auto tile = [&](const uint8_t* Ks, const uint8_t* Vs, float c, int rem, auto masked_tag) {
    constexpr bool kMasked = decltype(masked_tag)::value;
    // ---- S^T = K8 . Q8^T
    v16i S[4][QB];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) S[kb][qb][r] = 0;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int row = kb * 32 + l32;
        const v4i kf = *reinterpret_cast<const v4i*>(Ks + row * 128 + ((((4 * hh + m) ^ (row & 7)) & 7) << 4));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          S[kb][qb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf, qf[qb][m], S[kb][qb], 0, 0, 0);
      }
    }
    // ---- online softmax, P8 packing
    uint32_t P[QB][2][8];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      int mx = -(1 << 30);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (kMasked) {
            const int key = kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
            if (key >= rem) S[kb][qb][r] = -(1 << 30);
          }
          mx = max(mx, (int)S[kb][qb][r]);
        }
      mx = max(mx, other_half_i(mx));
      const float mt = (float)mx * c;
      const float mnew = fmaxf(m_run[qb], mt);
      if (__any(mnew > m_run[qb])) {
        const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - mnew);
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) O[db][qb][r] *= alpha;
      }
      m_run[qb] = mnew;
      const float mneg = kLog2_448 - mnew;
      float ls = 0.0f;
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int kb = 2 * g + (j >> 2);
          const int r0 = 4 * (j & 3);
          float pv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            pv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf((float)S[kb][qb][r0 + i], c, mneg));
            if (kMasked) {
              const int key = kb * 32 + 8 * (j & 3) + 4 * hh + i;
              if (key >= rem) pv[i] = 0.0f;
            }
            ls += pv[i];
          }
          int wd = __builtin_amdgcn_cvt_pk_fp8_f32(pv[0], pv[1], 0, false);
          wd = __builtin_amdgcn_cvt_pk_fp8_f32(pv[2], pv[3], wd, true);
          P[qb][g][j] = (uint32_t)wd;
        }
      l_run[qb] += ls;
    }
    // ---- O^T += V8^T . P8
#pragma unroll
    for (int g = 0; g < 2; ++g) {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int d = db * 32 + l32;
        const uint8_t* vrow = Vs + d * 128;
        const int ch0 = 4 * g + 2 * hh;
        const v4i lo = *reinterpret_cast<const v4i*>(vrow + (((ch0 ^ (d & 7)) & 7) << 4));
        const v4i hi = *reinterpret_cast<const v4i*>(vrow + ((((ch0 + 1) ^ (d & 7)) & 7) << 4));
        const v8i A = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const v8i Bp = {(int)P[qb][g][0], (int)P[qb][g][1], (int)P[qb][g][2], (int)P[qb][g][3],
                          (int)P[qb][g][4], (int)P[qb][g][5], (int)P[qb][g][6], (int)P[qb][g][7]};
          O[db][qb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, Bp, O[db][qb], 0, 0, 0, 127, 0, 127);
        }
      }
    }
  };


  gload(0);
  swrite(0);
  __syncthreads();
  for (int t = 0; t < p.nbk; ++t) {
    if (t + 1 < p.nbk) gload(t + 1);
    const uint8_t* Ks = smem + (t & 1) * kStageBytes;
    const uint8_t* Vs = Ks + kTileBytes;
    const float c = qscale * ksc[t] * p.sl2e;
    const int rem = p.Nkv - t * 128;
    if (rem >= 128) tile(Ks, Vs, c, rem, std::false_type{});
    else tile(Ks, Vs, c, rem, std::true_type{});
    if (t + 1 < p.nbk) swrite((t + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: O = acc * vs / l448 -> BF16
  const float* vsc = p.vs + bh * 128;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = l_run[qb] + other_half_f(l_run[qb]);
    const int q = q0 + 32 * qb + l32;
    if (q < p.Nq) {
      const float inv = 1.0f / lt;
      uint16_t* orow = p.out + b * p.os0 + (int64_t)q * p.os1 + h * p.os2;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int d0 = 32 * db + 8 * a + 4 * hh;
          const float4 sv = *reinterpret_cast<const float4*>(vsc + d0);
          const float o0 = O[db][qb][4 * a + 0] * sv.x * inv;
          const float o1 = O[db][qb][4 * a + 1] * sv.y * inv;
          const float o2 = O[db][qb][4 * a + 2] * sv.z * inv;
          const float o3 = O[db][qb][4 * a + 3] * sv.w * inv;
          *reinterpret_cast<uint2*>(orow + d0) =
              make_uint2(bf16_rne(o0) | (bf16_rne(o1) << 16), bf16_rne(o2) | (bf16_rne(o3) << 16));
        }
    }
  }
}

template <int QB, int NW>
hipError_t launch_cfg(const AttnArgs& a, hipStream_t stream) {
  const Layout& L = a.L;
  constexpr int BM = NW * QB * 32;
  AttnP p;
  p.q8 = a.packed + L.off_q8;
  p.k8 = a.packed + L.off_k8;
  p.v8 = a.packed + L.off_v8;
  p.qs = reinterpret_cast<const float*>(a.packed + L.off_qs);
  p.ks = reinterpret_cast<const float*>(a.packed + L.off_ks);
  p.vs = reinterpret_cast<const float*>(a.packed + L.off_vs);
  p.out = a.out;
  p.os0 = a.o_str[0];
  p.os1 = a.o_str[1];
  p.os2 = a.o_str[2];
  p.H = (int)L.H;
  p.Nq = (int)L.Nq;
  p.Nkv = (int)L.Nkv;
  p.nbq = (int)L.nbq;
  p.nbk = (int)L.nbk;
  p.mt = (int)((L.Nq + BM - 1) / BM);
  p.G = L.B * L.H * p.mt;
  p.sl2e = a.softmax_scale * kLog2e;
  const int64_t G8 = (p.G + 7) / 8 * 8;
  hipLaunchKernelGGL((attn_fwd_kernel<QB, NW>), dim3((unsigned)G8), dim3(NW * 64), kStageBytes * 2, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, bool cross, hipStream_t stream) {
  (void)cross;
  return launch_cfg<1, 4>(a, stream);
}

}  // namespace sattn
