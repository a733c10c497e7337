// attn_short.hip -- attention forward over short key sequences (at most 512
// keys, four 128-key tiles) for gfx950: persistent workgroups with the
// head's K/V codes resident in LDS.
//
// Text cross-attention in a diffusion transformer (the FA4 autotuning page,
// "Validation", covers cross- beside self-attention) has tens of thousands
// of queries against a few hundred text keys.  With a workgroup per
// 256-query tile, as in attn_fwd.hip, each workgroup runs only four tile
// steps, so its fixed costs -- loading the Q codes and the first K/V tiles,
// filling and draining the two-group pipeline, writing the output -- take
// about half of its time, and one workgroup per CU leaves nothing to hide
// them behind.  Here one workgroup per CU sweeps an equal share of the
// query tiles (in head order; a share that spans two heads runs them one
// after the other):
//   - the head's K and V^T tiles (128 KiB at most) are loaded into LDS once,
//     by LDS-DMA, and read by every query tile of the run;
//   - the two wave groups' MFMA / softmax alternation (see attn_fwd.hip)
//     runs on without a break from one query tile to the next: the MFMA
//     phase that finishes a tile's last P.V also starts the next tile's
//     Q.K^T and, between those MFMAs, writes half of the finished tile's
//     output; the next softmax phase, the tile's first (no rescale), writes
//     the other half;
//   - each wave's next Q codes are copied into LDS a whole query tile ahead.
// LDS: the K tiles (16 KiB each) in the first 64 KiB, the V^T tiles in the
// next 64 KiB, and 4 KiB per wave to stage its Q codes and output rows:
// 160 KiB.  Every K or V^T read is a lane constant plus an instruction
// offset below 64 KiB.  The arithmetic per tile is the dense kernel's:
// exact INT8 scores (or FP8 Q/K scores), the exact running maximum with the
// conditional rescale, P as E4M3(448 p), O in FP32.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
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
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2_448 = 8.80735492205760410744f;
constexpr int kNegInfBits = (int)0xFF800000u;
constexpr int kIntMin = (int)0x80000000u;
constexpr int kMaxTiles = 4;
constexpr int kVRegion = kMaxTiles * (int)kTileBytes;       // V^T tiles from 64 KiB
constexpr int kStageOut = 2 * kMaxTiles * (int)kTileBytes;  // per-wave output staging
constexpr int kLds = kStageOut + 8 * 4096;

struct ShortP {
  const uint8_t* q8;
  const uint8_t* k8;
  const uint8_t* v8;
  const float* qs;
  const float* ks;
  const float* vs;
  const float* km;
  uint16_t* out;
  int64_t os0, os1, os2;
  float* lse;
  int64_t BH;
  int H, Nq, Nkv, nbq, nbk, mt;
  int share, extra;  // B*H*mt query tiles = share * workgroups + extra
  float scale, sl2e;
};

__device__ inline int other_half_i(int x) {
  auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return (threadIdx.x & 32) ? (int)r[0] : (int)r[1];
}
__device__ inline float other_half_f(float x) { return __int_as_float(other_half_i(__float_as_int(x))); }

typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// two floats to BF16, rounded to nearest even, packed (v_cvt_pk_bf16_f32)
__device__ inline uint32_t bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f{lo, hi}), v2bf));
}

// lane N of each row of 16 lanes, to every lane of that row (DPP
// row_newbcast)
template <int N>
__device__ inline float row_bcast(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + N, 0xF, 0xF, false));
}

template <int I, int N, typename F>
__device__ inline void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// The lane index as a value the compiler must take as new at every use.
// The per-query-tile code (Q loads, output, LSE) derives its addresses from
// it, so they are recomputed once per query tile instead of being hoisted out
// of the tile loop and held -- or spilled -- across it.
__device__ inline int fresh_lane() {
  int l = (int)threadIdx.x;
  asm volatile("" : "+v"(l));
  return l & 63;
}

// A scalar the compiler must take as new at this point (kept in an SGPR):
// products formed from it in the per-query-tile code stay there instead of
// being hoisted and held across the tile loop.
template <typename T>
__device__ inline T fresh_s(T x) {
  asm volatile("" : "+s"(x));
  return x;
}

// A buffer resource over [base, base + bytes) for stores that drop every
// access past its end; base and bytes are the same in every lane (taken from
// the first, so that the compiler keeps the resource in scalar registers)
__device__ inline __amdgpu_buffer_rsrc_t uniform_rsrc(const void* base, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const int n = __builtin_amdgcn_readfirstlane(bytes);
  // word 3: 32-bit data format, no swizzle -- the range check then compares
  // byte offsets with the size
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0, n,
                                           0x00020000);
}

template <int OFF>
__device__ inline void copy_to_lds_off(const uint8_t* src_lane, uint8_t* dst_wave) {
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src_lane,
                                   (void __attribute__((address_space(3)))*)dst_wave, 16, OFF, 0);
}

// NBK: key tiles of a head (1..4), a template parameter so that every tile's
// LDS addresses are lane constants plus immediates.  LSE: the per-row LSE is
// written too (the instances without it carry none of its code).  TAIL: the
// last key tile is partial (Nkv not a multiple of 128); without it the
// instance carries no masking code, whose registers would otherwise be
// reserved across the whole tile loop.
// One run of a workgroup: query tiles [t_lo, t_hi) of head bh, with the
// head's K and V^T loaded into LDS first.
template <bool FP8QK, int NBK, bool LSE, bool TAIL>
__device__ __attribute__((always_inline)) inline void short_run(const ShortP& p, const int64_t bh, const int t_lo,
                                                                const int t_hi) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int64_t b = bh / p.H, h = bh % p.H;
  // the head's pointers, formed once: the loop reads no other kernel
  // argument, so the rest need no registers across it
  const uint8_t* const qhead = p.q8 + bh * p.nbq * kTileBytes;
  // (the Q and K block scales through the constant address space: scalar
  // loads, counted apart from the vector memory operations, so that a use of
  // one never waits for the output's stores)
  const __attribute__((address_space(4))) float* const qsh =
      (const __attribute__((address_space(4))) float*)(p.qs + bh * p.nbq);
  const float* const kmh = p.km + bh * 128;
  uint16_t* const outh = p.out + b * p.os0 + h * p.os2;
  float* const lseh = LSE ? p.lse + bh * p.Nq : nullptr;
  const int64_t os1 = p.os1;
  const int Nq = p.Nq, nbq = p.nbq;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const bool isA = w < 4;
  const int rem = p.Nkv - (NBK - 1) * 128;  // keys in the last tile
  const __attribute__((address_space(4))) float* ksc4 =
      (const __attribute__((address_space(4))) float*)(p.ks + bh * NBK);
  uint8_t* obuf = smem + kStageOut + w * 4096;  // this wave's 4 KiB

  auto barrier = [] {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // The wave's 32 rows of Q codes of query tile mt (4 KiB, contiguous in
  // the packed Q tile) into its staging area by LDS-DMA; false when the
  // rows lie past the last Q block (their codes are then zero).
  auto q_dma = [&](int mt) __attribute__((always_inline)) -> bool {
    const int q0 = mt * 256 + w * 32;
    if (q0 >= nbq * 128) return false;
    const uint8_t* src = qhead + (q0 >> 7) * kTileBytes + (q0 & 127) * 128 + fresh_lane() * 16;
    copy_to_lds_off<0>(src, obuf);
    copy_to_lds_off<1024>(src, obuf);
    copy_to_lds_off<2048>(src, obuf);
    copy_to_lds_off<3072>(src, obuf);
    return true;
  };

  v4i qf[4];
  float qscale = 0.0f;
  float m_run = -__builtin_inff(), l_run = 0.0f;
  v16f O[4];
  v16i S[4];
  uint32_t P[2][8];
  float c_cur = 0.0f;

  // the codes of query tile mt from the staging area (lane: row l32, bytes
  // 64 hh .. 64 hh + 63), after the wave's DMA of them has completed
  auto q_read = [&](int mt, bool valid) __attribute__((always_inline)) {
    const int q0 = mt * 256 + w * 32;
    if (valid) {
      const int ln = fresh_lane();
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
      for (int m = 0; m < 4; ++m) qf[m] = *reinterpret_cast<const v4i*>(obuf + (ln & 31) * 128 + 64 * (ln >> 5) + 16 * m);
      qscale = qsh[q0 >> 7];
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m) qf[m] = v4i{0, 0, 0, 0};
      qscale = 0.0f;
    }
  };

  // softmax_scale * qs * sum_d qcode_d kmean_d: the LSE's smoothing shift of
  // the wave's current rows (from the Q codes this lane holds: channels
  // 64 hh + 16 m + 4 j + e).  The K means come four per lane, as the V
  // scales do below: lane 16 r + n of kmx[m] holds the mean of channel
  // 64 (r >> 1) + 16 m + n, and a broadcast of lane 4 j + e within each row
  // of 16 lanes gives every lane the mean of its channel.
  auto lse_shift = [&]() __attribute__((always_inline)) -> float {
    const int ln = fresh_lane();
    const float* kml = kmh + 64 * (ln >> 5) + (ln & 15);
    float kmx[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) kmx[m] = kml[16 * m];
    float acc = 0.0f;
#pragma unroll
    for (int m = 0; m < 4; ++m)
      static_for<0, 4>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        const int word = qf[m][j];
        float qc[4];
        if constexpr (FP8QK) {
          qc[0] = __builtin_amdgcn_cvt_f32_fp8(word, 0);
          qc[1] = __builtin_amdgcn_cvt_f32_fp8(word, 1);
          qc[2] = __builtin_amdgcn_cvt_f32_fp8(word, 2);
          qc[3] = __builtin_amdgcn_cvt_f32_fp8(word, 3);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) qc[e] = (float)(int8_t)(word >> (8 * e));
        }
        acc = __builtin_fmaf(qc[0], row_bcast<4 * j + 0>(kmx[m]), acc);
        acc = __builtin_fmaf(qc[1], row_bcast<4 * j + 1>(kmx[m]), acc);
        acc = __builtin_fmaf(qc[2], row_bcast<4 * j + 2>(kmx[m]), acc);
        acc = __builtin_fmaf(qc[3], row_bcast<4 * j + 3>(kmx[m]), acc);
      });
    acc += other_half_f(acc);
    return p.scale * qscale * acc;
  };

  // The head's V scales for the output, four per lane: lane 16 r + n of
  // vsx[db] holds vs[32 db + 8 (n >> 2) + (n & 3) + 4 (r >> 1)], so that a
  // broadcast of lane 4 a + j within each row of 16 lanes gives every lane
  // the scale of its output channel 32 db + 8 a + 4 hh + j.
  float vsx[4];
  {
    const int ln = fresh_lane();
    const float* vsr = p.vs + bh * 128 + 8 * ((ln & 15) >> 2) + (ln & 3) + 4 * (ln >> 5);
#pragma unroll
    for (int db = 0; db < 4; ++db) vsx[db] = vsr[32 * db];
  }

  // ---- output of the wave's 32 rows of query tile mt: O = acc * vs /
  // l448 -> BF16 through the staging area (whole 128-byte lines per
  // store), and the LSE
  // The stores are buffer stores whose range ends after the last row that
  // exists (no row at all before the first tile, write = false): rows past
  // Nq are dropped by the hardware's range check instead of by branches, so
  // the whole output is one block of straight-line code that the compiler
  // can interleave with the Q.K^T MFMAs issued before it.  (The arithmetic
  // runs before the first tile too, so that the P.V products it consumes
  // are not sunk into a conditional block.)
  // Halves [h_lo, h_hi) of the rows' channels (half h: O blocks 2h, 2h+1);
  // inv = 1 / l448 of the rows, taken before the next tile resets l.  The
  // LSE goes out with half 0, while m and l are still the tile's.
  auto epilogue = [&](int mt, float shift, bool write, int h_lo, int h_hi, float inv) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 2 * h_lo; db < 2 * h_hi; ++db) asm volatile("" : "+v"(O[db]));
    const int q0 = mt * 256 + w * 32;
    const int ln = fresh_lane(), el32 = ln & 31, ehh = ln >> 5;
    // the staging area's rows go out as 16-byte chunks: lane ln stores chunk
    // cc of rows 8 i + rr
    const int rr = ln >> 3, cc = ln & 7;
    const int64_t os1f = fresh_s(os1);
    const int rb = 2 * (int)os1f;  // bytes from one query row to the next
    const int nq_left = max(0, min(32, fresh_s(Nq) - q0));
    const int nrows = write ? nq_left : 0;
    const __amdgpu_buffer_rsrc_t orsrc =
        uniform_rsrc(fresh_s(outh) + (int64_t)q0 * os1f, nrows > 0 ? (nrows - 1) * rb + 256 : 0);
    const int ooff = rr * rb + 16 * cc;
#pragma unroll
    for (int half = h_lo; half < h_hi; ++half) {
      asm volatile("" ::: "memory");
#pragma unroll
      for (int db2 = 0; db2 < 2; ++db2) {
        const int db = 2 * half + db2;
        static_for<0, 4>([&](auto ac) {
          constexpr int a = decltype(ac)::value;
          // channel 32 db + 8 a + 4 hh + j of this lane's row
          const float o0 = O[db][4 * a + 0] * inv * row_bcast<4 * a + 0>(vsx[db]);
          const float o1 = O[db][4 * a + 1] * inv * row_bcast<4 * a + 1>(vsx[db]);
          const float o2 = O[db][4 * a + 2] * inv * row_bcast<4 * a + 2>(vsx[db]);
          const float o3 = O[db][4 * a + 3] * inv * row_bcast<4 * a + 3>(vsx[db]);
          const int c = 4 * db2 + a;
          *reinterpret_cast<uint2*>(obuf + el32 * 128 + (((c ^ swz(el32)) & 7) << 4) + 8 * ehh) =
              make_uint2(bf16x2(o0, o1), bf16x2(o2, o3));
        });
      }
      v4i val[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 8 * i + rr;
        val[i] = *reinterpret_cast<const v4i*>(obuf + r * 128 + (((cc ^ swz(r)) & 7) << 4));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_raw_buffer_store_b128(val[i], orsrc, ooff + 8 * i * rb + 128 * half, 0, 0);
    }
    if (LSE && h_lo == 0) {
      const float lt = l_run + other_half_f(l_run);
      // the LSE of row el32 from the lanes of half 0 (the others' offset is
      // past the range)
      const __amdgpu_buffer_rsrc_t lrsrc = uniform_rsrc(lseh + q0, 4 * nrows);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(kLn2 * (m_run + log2f(lt) - kLog2_448) + shift),
                                            lrsrc, ehh == 0 ? 4 * el32 : 128, 0, 0);
    }
    // the staging reads are complete before the area is written again
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };

  // (O needs no clearing: the query tile's first P.V starts from zero)
  auto reset = [&] {
    m_run = -__builtin_inff();
    l_run = 0.0f;
  };

  // Lane constants of the LDS reads.  K: row kb*32 + l32 of a tile, logical
  // chunk 4 hh + m; V^T: row db*32 + l32, chunks 4 g + 2 hh and 4 g + 2 hh + 1.
  // The rows' swizzle (row >> 1) & 7 does not depend on kb or db, which go
  // with the tile into the instructions' immediate offsets.  The V^T
  // region's base is part of the V^T lane constants: the rest of a V^T
  // address (tile and row block, below 64 KiB) then fits the offset field.
  int koff[4], voff[2][2];
#pragma unroll
  for (int m = 0; m < 4; ++m) koff[m] = l32 * 128 + ((((4 * hh + m) ^ swz(l32)) & 7) << 4);
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int x = 0; x < 2; ++x) voff[g][x] = kVRegion + l32 * 128 + ((((4 * g + 2 * hh + x) ^ swz(l32)) & 7) << 4);

  // ---- M phase pieces: P.V of tile tp (its P in registers), S of tile t.
  // (tp = 0: the query tile's first P.V, into zero accumulators)
  auto pv = [&](int tp) __attribute__((always_inline)) {
    const uint8_t* Vs = smem + tp * kTileBytes;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const v8i Bp = {(int)P[g][0], (int)P[g][1], (int)P[g][2], (int)P[g][3],
                      (int)P[g][4], (int)P[g][5], (int)P[g][6], (int)P[g][7]};
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const v4i lo = *reinterpret_cast<const v4i*>(Vs + db * 4096 + voff[g][0]);
        const v4i hi = *reinterpret_cast<const v4i*>(Vs + db * 4096 + voff[g][1]);
        const v8i A = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        O[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, Bp, tp == 0 && g == 0 ? v16f{} : O[db], 0, 0,
                                                                 0, 127, 0, 127);
      }
    }
  };
  auto kread = [&](const uint8_t* Ks, int kb, int m) __attribute__((always_inline)) -> v4i {
    return *reinterpret_cast<const v4i*>(Ks + kb * 4096 + koff[m]);
  };
  // masked: tile t is the last one and holds rem < 128 keys; the others get
  // the integer minimum (INT8) or -inf (FP8 Q/K).  lean: the K operands are
  // read from LDS a quarter at a time (the empty asm with a memory clobber
  // keeps the next quarter's reads behind it), for the last key tile, whose
  // phase also takes the LSE shift and so has fewer registers to spare.
  auto scores = [&](int t, bool masked, bool lean) __attribute__((always_inline)) {
    const uint8_t* Ks = smem + t * kTileBytes;
    if constexpr (FP8QK) {
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          if (lean && (kb & 1) == 0) asm volatile("" ::: "memory");
          const v4i a0 = kread(Ks, kb, 2 * c), a1 = kread(Ks, kb, 2 * c + 1);
          const v4i b0 = qf[2 * c], b1 = qf[2 * c + 1];
          const v8i A = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
          const v8i Bq = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
          const v16f acc = c == 0 ? v16f{} : __builtin_bit_cast(v16f, S[kb]);
          S[kb] = __builtin_bit_cast(
              v16i, __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, Bq, acc, 0, 0, 0, 127, 0, 127));
        }
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        if (lean) asm volatile("" ::: "memory");
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          S[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kread(Ks, kb, m), qf[m], m == 0 ? v16i{} : S[kb], 0, 0, 0);
      }
    }
    c_cur = qscale * ksc4[t] * p.sl2e;
    if (masked) {
      int rl = rem - 4 * (fresh_lane() >> 5);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          asm volatile("" : "+v"(rl));
          if (kb * 32 + 8 * (r >> 2) + (r & 3) >= rl) S[kb][r] = FP8QK ? kNegInfBits : kIntMin;
        }
    }
  };

  auto score_f = [&](int s) __attribute__((always_inline)) -> float {
    if constexpr (FP8QK) return __int_as_float(s);
    else return (float)s;
  };
  // INT8 scores of masked keys hold the integer minimum: that keeps them out
  // of the row maximum, and their p, all equal, is taken back out of l below.
  // Their P codes multiply V^T columns that are zero past the last key, so
  // they add nothing to O.  (FP8 Q/K scores of masked keys are -inf: p = 0.)
  // Keys of lane half hh: k in [0, 128) with bit 2 of k equal to hh.
  // (computed where it is used, once per query tile: held across the
  // sweep it would only take a register)
  auto nmask = [&]() __attribute__((always_inline)) -> float {
    int r = rem;
    asm volatile("" : "+s"(r));
    const int part = r & 7;
    const int below = 4 * (r >> 3) + ((fresh_lane() >> 5) == 0 ? min(part, 4) : max(part - 4, 0));
    return (float)(64 - below);
  };

  // ---- V phase: online softmax of S -> P with the conditional rescale of O
  // (first: the query tile's first key tile, where m = -inf and O = 0)
  auto vblock = [&](bool first, bool masked) __attribute__((always_inline)) {
    (void)masked;
    const float c = c_cur == 0.0f ? 1.17549435e-38f : c_cur;
    float mt;
    if constexpr (FP8QK) {
      float mx = -__builtin_inff();
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, __int_as_float(S[kb][r]));
      mx = fmaxf(mx, other_half_f(mx));
      mt = mx * c;
    } else {
      int mx = kIntMin;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = max(mx, (int)S[kb][r]);
      mx = max(mx, other_half_i(mx));
      mt = (float)mx * c;
    }
    const float mnew = fmaxf(m_run, mt);
    if (!first && __any(mnew > m_run)) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - mnew);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) O[db][r] *= alpha;
    }
    m_run = mnew;
    const float nb = kLog2_448 - mnew;
    float ls[4];
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int kb = 2 * g + (j >> 2);
        const int r0 = 4 * (j & 3);
        float pvv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pvv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(score_f(S[kb][r0 + i]), c, nb));
          ls[i] = (g == 0 && j == 0) ? pvv[i] : ls[i] + pvv[i];
        }
        // the first conversion writes the low half only: start from the
        // register's old contents instead of materialising a zero (not in
        // the instances with a partial tile, where holding them costs spills)
        int wd = __builtin_amdgcn_cvt_pk_fp8_f32(pvv[0], pvv[1], TAIL ? 0 : (int)P[g][j], false);
        wd = __builtin_amdgcn_cvt_pk_fp8_f32(pvv[2], pvv[3], wd, true);
        P[g][j] = (uint32_t)wd;
      }
    l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);
    if constexpr (!FP8QK) {
      if (masked) l_run -= nmask() * __builtin_amdgcn_exp2f(__builtin_fmaf((float)kIntMin, c, nb));
    }
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int j = 0; j < 8; ++j) asm volatile("" ::"v"(P[g][j]));
    asm volatile("" ::"v"(l_run));
  };

#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int j = 0; j < 8; ++j) P[g][j] = 0u;

  // prologue: the head's K and V^T tiles into LDS (waves 0-3 copy 4 KiB each
  // of every K tile, waves 4-7 of every V^T tile) and the first query
  // tile's codes into each wave's staging area
  {
    const uint8_t* src0 = (w < 4 ? p.k8 : p.v8) + bh * NBK * kTileBytes + (w & 3) * 4096 + fresh_lane() * 16;
    uint8_t* dst0 = smem + (w < 4 ? 0 : kVRegion) + (w & 3) * 4096;
#pragma unroll
    for (int t = 0; t < NBK; ++t) {
      copy_to_lds_off<0>(src0 + t * kTileBytes, dst0 + t * kTileBytes);
      copy_to_lds_off<1024>(src0 + t * kTileBytes, dst0 + t * kTileBytes);
      copy_to_lds_off<2048>(src0 + t * kTileBytes, dst0 + t * kTileBytes);
      copy_to_lds_off<3072>(src0 + t * kTileBytes, dst0 + t * kTileBytes);
    }
  }
  bool qvalid = q_dma(t_lo);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  // With two key tiles or more, a query tile's codes are read from the
  // staging area during its predecessor's last M phase (the first tile's
  // here), and its LSE shift is taken there before they are replaced.
  if constexpr (NBK > 1) q_read(t_lo, qvalid);
  float shift = 0.0f;
  m_run = -__builtin_inff();
  l_run = 0.0f;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) O[db][r] = 0.0f;

  // the ping-pong over query tiles and their key tiles; group B runs one
  // barrier slot behind group A
  if (!isA) barrier();
  float shift_prev = 0.0f, inv_prev = 0.0f;
  for (int mt = t_lo; mt < t_hi; ++mt) {
#pragma unroll
    for (int t = 0; t < NBK; ++t) {
      // M phase
      __builtin_amdgcn_s_setprio(2);
      // (TAIL implies rem < 128; the run-time test keeps the masking code in
      // a branch of its own, which in the one-tile instances avoids spills)
      const bool masked = TAIL && t == NBK - 1 && rem < 128;
      if (t > 0) {
        pv(t - 1);
        scores(t, masked, t == NBK - 1);
        // the S MFMAs of this tile are issued: its LSE shift, from its codes
        if (LSE && t == NBK - 1) shift = lse_shift();
      } else {
        // the previous query tile's last P.V (P = 0 before the first tile)
        // and this tile's first S; then, while those MFMAs run, the first
        // half of the previous tile's output through the staging area (the
        // second half follows in this tile's first softmax phase, which has
        // no rescale to do)
        pv(NBK - 1);
        shift_prev = shift;
        if constexpr (NBK == 1) {
          // (one key tile: this tile's codes are read here)
          if (LSE && mt > t_lo) shift_prev = lse_shift();
          q_read(mt, qvalid);
        }
        // the P.V products complete here: the empty asm keeps them ahead of
        // the Q.K^T MFMAs, which would otherwise be free to go first and make
        // the output wait for both
#pragma unroll
        for (int db = 0; db < 4; ++db) asm volatile("" : "+v"(O[db]));
        __builtin_amdgcn_sched_barrier(0);
        scores(0, masked, false);
        inv_prev = 1.0f / (l_run + other_half_f(l_run));
        epilogue(mt - 1, shift_prev, mt > t_lo, 0, 1, inv_prev);
        // a wave issues in order: each Q.K^T MFMA followed by a share of the
        // output's VALU work, which then runs while the MFMA does
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        reset();
      }
      // The phase's MFMAs are issued before the barrier: without these uses
      // the compiler is free to sink them (their results are needed only
      // later) into the V phase, where they would compete with the partner
      // group's MFMAs.
#pragma unroll
      for (int db = 0; db < 4; ++db) asm volatile("" ::"v"(O[db]));
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) asm volatile("" ::"v"(S[kb]));
      __builtin_amdgcn_s_setprio(0);
      barrier();
      // V phase (with two key tiles or more, the last one first reads the
      // next query tile's codes, copied into the staging area a tile ago;
      // the first one writes the second half of the previous tile's output,
      // then starts the copy of the next tile's codes into the staging area)
      if (NBK > 1 && t == NBK - 1 && mt + 1 < t_hi) q_read(mt + 1, qvalid);
      if (t == 0) {
        epilogue(mt - 1, shift_prev, mt > t_lo, 1, 2, inv_prev);
        if (mt + 1 < t_hi) qvalid = q_dma(mt + 1);
      }
      vblock(t == 0, masked);
      barrier();
    }
  }
  // the last query tile's P.V and output
  pv(NBK - 1);
  if constexpr (LSE && NBK == 1) shift = lse_shift();
  epilogue(t_hi - 1, shift, true, 0, 2, 1.0f / (l_run + other_half_f(l_run)));
  if (isA) barrier();
}

// The B*H*mt query tiles, in head order, are cut into p.groups equal
// contiguous shares, one per workgroup (one workgroup per CU); a share that
// spans heads is run head by head, reloading K and V^T in between.
template <bool FP8QK, int NBK, bool LSE, bool TAIL>
__global__ __launch_bounds__(512, 1) void attn_short_kernel(ShortP p) {
  // the first p.extra workgroups take p.share + 1 tiles, the rest p.share
  const int g = blockIdx.x;
  int lo = g * p.share + min(g, p.extra);
  const int hi = lo + p.share + (g < p.extra ? 1 : 0);
  for (bool first = true; lo < hi; first = false) {
    const int mt = fresh_s(p.mt);
    const int bh = lo / mt;
    const int t_lo = lo - bh * mt;
    const int t_hi = min(mt, t_lo + (hi - lo));
    // the previous run's reads of the K/V^T and staging areas are complete
    // before this run's copies overwrite them
    if (!first) __syncthreads();
    short_run<FP8QK, NBK, LSE, TAIL>(p, bh, t_lo, t_hi);
    lo += t_hi - t_lo;
  }
}

int cu_count() {
  static std::atomic<int> n{0};
  int v = n.load(std::memory_order_relaxed);
  if (v == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    n.store(v, std::memory_order_relaxed);
  }
  return v;
}

template <bool FP8QK, int NBK, bool LSE, bool TAIL>
hipError_t launch_short(const AttnArgs& a, hipStream_t stream) {
  const Layout& L = a.L;
  constexpr int kMaxDev = 64;
  static std::atomic<bool> attr_set[kMaxDev];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev || !attr_set[dev].load(std::memory_order_acquire)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_short_kernel<FP8QK, NBK, LSE, TAIL>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kMaxDev) attr_set[dev].store(true, std::memory_order_release);
  }
  ShortP p;
  p.q8 = a.packed + L.off_q8;
  p.k8 = a.packed + L.off_k8;
  p.v8 = a.packed + L.off_v8;
  p.qs = reinterpret_cast<const float*>(a.packed + L.off_qs);
  p.ks = reinterpret_cast<const float*>(a.packed + L.off_ks);
  p.vs = reinterpret_cast<const float*>(a.packed + L.off_vs);
  p.km = reinterpret_cast<const float*>(a.packed + L.off_km);
  p.out = a.out;
  p.os0 = a.o_str[0];
  p.os1 = a.o_str[1];
  p.os2 = a.o_str[2];
  p.lse = a.lse;
  p.BH = L.B * L.H;
  p.H = (int)L.H;
  p.Nq = (int)L.Nq;
  p.Nkv = (int)L.Nkv;
  p.nbq = (int)L.nbq;
  p.nbk = (int)L.nbk;
  p.mt = (int)((L.Nq + 255) / 256);
  // one workgroup per CU, each with an equal share of the query tiles
  const int64_t total = p.BH * p.mt;
  const int64_t groups = min((int64_t)cu_count(), total);
  p.share = (int)(total / groups);
  p.extra = (int)(total % groups);
  p.scale = a.softmax_scale;
  p.sl2e = a.softmax_scale * kLog2e;
  const int64_t grid = groups;
  hipLaunchKernelGGL((attn_short_kernel<FP8QK, NBK, LSE, TAIL>), dim3((unsigned)grid), dim3(512), kLds, stream, p);
  return hipGetLastError();
}

}  // namespace

bool short_kv_applies(const AttnArgs& a) {
  // (output rows at least one row of channels apart and 32 rows within
  // the 32-bit offsets of the epilogue's buffer stores)
  // (and the tile count in 32 bits)
  return a.lut_counts == nullptr && !a.L.qsmooth && a.splits == 1 && a.L.nbk >= 1 && a.L.nbk <= kMaxTiles &&
         a.L.B * a.L.H * ((a.L.Nq + 255) / 256) < ((int64_t)1 << 30) &&
         a.o_str[1] >= 128 && a.o_str[1] < ((int64_t)1 << 24) &&
         a.L.B * a.L.H * ((a.L.Nq + 255) / 256) > (int64_t)cu_count();
}

template <bool FP8QK, bool LSE, bool TAIL>
hipError_t launch_short_nbk(const AttnArgs& a, hipStream_t stream) {
  switch (a.L.nbk) {
    case 1: return launch_short<FP8QK, 1, LSE, TAIL>(a, stream);
    case 2: return launch_short<FP8QK, 2, LSE, TAIL>(a, stream);
    case 3: return launch_short<FP8QK, 3, LSE, TAIL>(a, stream);
    case 4: return launch_short<FP8QK, 4, LSE, TAIL>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <bool FP8QK, bool LSE>
hipError_t launch_short_tail(const AttnArgs& a, hipStream_t stream) {
  return a.L.Nkv % 128 != 0 ? launch_short_nbk<FP8QK, LSE, true>(a, stream)
                            : launch_short_nbk<FP8QK, LSE, false>(a, stream);
}

hipError_t launch_attention_short(const AttnArgs& a, hipStream_t stream) {
  if (a.lse != nullptr)
    return a.fp8qk ? launch_short_tail<true, true>(a, stream) : launch_short_tail<false, true>(a, stream);
  return a.fp8qk ? launch_short_tail<true, false>(a, stream) : launch_short_tail<false, false>(a, stream);
}

}  // namespace sattn
