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
// (two groups of waves alternate MFMA and softmax phases; K/V tiles stream
// into three LDS stages by LDS-DMA while earlier tiles are consumed).
//
// Data flow per wave (32 queries; 128-key tiles):
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
//   epilogue          O = acc * vs[d] / l448, BF16 round-to-nearest-even;
//                     optionally the row's log-sum-exp (FP32, natural log).
//
// attn_pp_kernel<true> is the FP8 Q/K format (the FP8/FP8/BF16 row of the MHA
// v4 page's MI355X table): Q and K codes are E4M3, S^T comes from the FP8
// MFMA (two 32x32x64 per 32-key block) as floats, and the row max is a float
// max.  That instruction does not round its 64-product sum correctly: its
// error grows with the spread of the products' exponents, up to about 2^-12
// of the sum of their magnitudes, while the INT8 one is exact.
//
// Split-KV (the FA4 autotuning page's split-KV with an FP32 LSE): a launch may
// give each workgroup a range of a head's key tiles; it then writes its FP32
// output and LSE to a workspace, and k_combine merges the ranges by the
// log-sum-exp rule.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

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
constexpr int kStageBytes = 2 * (int)kTileBytes;  // K tile + V^T tile

struct AttnP {
  const uint8_t* q8;
  const uint8_t* k8;
  const uint8_t* v8;
  const float* qs;
  const float* ks;
  const float* vs;
  const float* km;  // K mean [B*H][128]
  uint16_t* out;
  int64_t os0, os1, os2;
  float* lse;    // [B*H][Nq] or null
  float* opart;  // split partials: FP32 O [splits][B*H][Nq][128] (splits > 1)
  float* lpart;  //   and their LSE [splits][B*H][Nq]
  const int32_t* lut_counts;    // block-sparse: key tiles per query tile [B*H*mt]
  const uint32_t* lut_entries;  //   and their entries [B*H*mt][nbk]
  const float* ds;              // Q smoothing, E4M3 codes: Delta-S [B*H][nbq][nbk*128]
  const int8_t* dg;             //   INT8 codes: digit rows of mean / unit [B*H][nbq][4][128]
  const float* dp;              //   and their parameters [B*H][nbq][8]
  const float* qm;              //   the Q block means [B*H][nbq][128]
  int64_t G;     // logical workgroups: B*H*splits*mt
  int64_t BH;
  int H, Nq, Nkv, nbq, nbk, mt;
  int splits, tps;  // key-tile ranges [s*tps, min(nbk, (s+1)*tps)) per split s
  float scale;      // softmax_scale
  float sl2e;       // softmax_scale * log2(e)
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

// MFMAs read their operands from all 64 lanes.  The epilogue stores under a
// per-lane condition (rows past Nq), and without this fence the compiler may
// sink the last PV MFMAs into that exec-masked region, where masked-off
// lanes would feed wrong operands into the valid lanes' results.  The empty
// asm "reads and rewrites" the accumulators, so they are complete before the
// branch.
__device__ inline void pin_accumulators(v16f (&O)[4]) {
#pragma unroll
  for (int db = 0; db < 4; ++db) asm volatile("" : "+v"(O[db]));
}

// Global -> LDS copy of one 16-byte piece per lane (global_load_lds with
// 16-byte size, new on gfx950): lane l's piece lands at dst + OFF + 16 l, so
// each wave instruction fills 1 KiB of LDS without passing through VGPRs.
// OFF (the instruction's immediate offset) is added to both addresses.
template <int OFF>
__device__ inline void copy_to_lds_off(const uint8_t* src_lane, uint8_t* dst_wave) {
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src_lane,
                                   (void __attribute__((address_space(3)))*)dst_wave, 16, OFF, 0);
}

// Masked keys of the last tile: the bits of -inf (FP8 Q/K scores are
// floats) or the integer minimum (INT8 scores, below every score, so the
// integer row maximum ignores it; the softmax of that tile maps it to -inf).
constexpr int kNegInfBits = (int)0xFF800000u;
constexpr int kIntMin = (int)0x80000000u;

// ---------------------------------------------------------------------------
// 8 waves, 32 queries each.  Waves w and w+4 share a SIMD.
// Group A (waves 0-3) runs one barrier slot ahead of group B (waves 4-7), so
// in every slot one wave of each SIMD issues MFMAs while its partner runs the
// softmax on the VALU:
//     slot    2t          2t+1        2t+2
//     A       M(t)        V(t)        M(t+1)
//     B       V(t-1)      M(t)        V(t)
// M(t) = O += V(t-1)^T . P(t-1) followed by S(t) = K(t) . Q^T;
// V(t) = online softmax of S(t) -> P(t), with the conditional O rescale.
// Tile u lives in LDS stage u % 3 from slot 2u (K read by A) to slot 2u+3
// (V read by B).  Tile t+1 is loaded in halves: its K tile by group A at the
// start of A's M(t), waited for at the end of A's V(t); its V^T tile by
// group B at the start of B's M(t), waited for at the end of B's V(t).
// (INT8 Q smoothing: four stages, tile t+2 loaded in M(t), whose waves also
// form Delta-S of tile t+1.)
// FP8QK: Q and K codes are E4M3 (the FP8/FP8/BF16 format): S^T comes from
// v_mfma_scale_f32_32x32x64_f8f6f4 in FP32, the K operands being the same
// LDS reads taken two 16-byte chunks per MFMA.
// QSMOOTH: Q was smoothed per block; each score gets the Delta-S term of its
// query block and key.  INT8 codes: the wave forms it in its MFMA phase from
// the block's digit rows and the K operands it already holds (16 more INT8
// MFMAs), rounds it to the accumulator unit and starts the score
// accumulators from it, so the softmax phase is the unsmoothed one.  E4M3
// codes: a table staged with the tile (1 KiB: the two query blocks' 128
// values) in LDS, added to each score in the softmax phase.
template <bool FP8QK, bool SPARSE, bool QSMOOTH>
__global__ __launch_bounds__(512, 1) void attn_pp_kernel(AttnP p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr bool DS_MFMA = QSMOOTH && !FP8QK;   // Delta-S from digit rows, in the accumulator
  constexpr bool DS_TABLE = QSMOOTH && FP8QK;   // Delta-S from the table, added per score
  constexpr int kStage = kStageBytes + (DS_TABLE ? 1024 : 0);
  // K/V stages, and how far ahead group A loads: INT8 Q smoothing forms a
  // tile's Delta-S one tile ahead, so it keeps four stages and loads two
  // tiles ahead
  constexpr int NS = DS_MFMA ? 4 : 3;
  constexpr int PD = NS - 2;
  // INT8 Q smoothing, beyond the stages: per group, Delta-S of two tiles
  // (by tile parity, 128 ints each), then per group its block's digit rows
  constexpr int kDsOff = NS * kStage;
  constexpr int kDigOff = kDsOff + 2048;
  constexpr int NW = 8;
  constexpr int BM = NW * 32;

  const int64_t G8 = (p.G + 7) / 8 * 8;
  const int64_t wg = blockIdx.x;
  const int64_t L = (wg % 8) * (G8 / 8) + wg / 8;
  if (L >= p.G) return;
  // logical order (b, h, split, query tile), query tile fastest: the
  // workgroups sharing one K/V range are consecutive, hence on one XCD
  const int64_t bhs = L / p.mt;
  const int mtile = (int)(L % p.mt);
  const int64_t bh = bhs / p.splits;
  const int split = (int)(bhs % p.splits);
  const int64_t b = bh / p.H, h = bh % p.H;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // the wave index through readfirstlane: a scalar, so every branch on the
  // wave's group (and the barriers inside them) is a scalar branch
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const bool isA = w < 4;
  const int q0 = mtile * BM + w * 32;
  const int qblk = q0 >> 7;
  // this workgroup's key tiles: [t0, t0 + nbk) of the head's p.nbk, nbk >= 1;
  // block-sparse: the nbk >= 0 tiles its LUT entries list (t0 = 0)
  const int t0 = split * p.tps;
  int nbk = min(p.nbk - t0, p.tps);
  const __attribute__((address_space(4))) uint32_t* ent = nullptr;
  if constexpr (SPARSE) {
    // scalar loads; a count or index out of range is clamped, so a
    // malformed table cannot make the kernel read outside the head
    const __attribute__((address_space(4))) int32_t* cnt =
        (const __attribute__((address_space(4))) int32_t*)(p.lut_counts);
    nbk = min(max(cnt[L], 0), p.nbk);
    ent = (const __attribute__((address_space(4))) uint32_t*)(p.lut_entries) + L * p.nbk;
    if (nbk == 0) {  // no allowed key for either query block: O = 0, lse = -inf
      const int q = q0 + l32;
      if (q < p.Nq) {
        uint16_t* orow = p.out + b * p.os0 + (int64_t)q * p.os1 + h * p.os2;
#pragma unroll
        for (int a = 0; a < 8; ++a) *reinterpret_cast<uint4*>(orow + 64 * hh + 8 * a) = make_uint4(0, 0, 0, 0);
        if (p.lse != nullptr && hh == 0) p.lse[bh * p.Nq + q] = -__builtin_inff();
      }
      return;
    }
  }
  // key tile of local step t, and whether this wave group's query block
  // attends it (entry bit 30: the tile's first 128 queries, waves 0-3; bit
  // 31: the second 128, waves 4-7)
  auto tile_of = [&](int t) __attribute__((always_inline)) -> int {
    if constexpr (SPARSE) return min((int)(ent[t] & 0x3FFFFFFFu), p.nbk - 1);
    else return t;
  };
  auto group_attends = [&](int t) __attribute__((always_inline)) -> bool {
    if constexpr (SPARSE) return ((ent[t] >> (isA ? 30 : 31)) & 1u) != 0;
    else return true;
  };

  v4i qf[4];
  float qscale = 0.0f;
  // INT8 Q smoothing: the weights of the block's four digit rows (the rows
  // themselves go to LDS below)
  float dw[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  v4i dgr[4];  // the digit rows as the A operand, read from LDS once
  if (q0 < p.nbq * 128) {
    const uint8_t* qt = p.q8 + (bh * p.nbq + qblk) * kTileBytes;
    const v4i* src = reinterpret_cast<const v4i*>(qt + ((q0 & 127) + l32) * 128 + 64 * hh);
#pragma unroll
    for (int m = 0; m < 4; ++m) qf[m] = src[m];
    qscale = p.qs[bh * p.nbq + qblk];
    if constexpr (DS_MFMA) {
      const __attribute__((address_space(4))) float* prm =
          (const __attribute__((address_space(4))) float*)(p.dp) + (bh * p.nbq + qblk) * kDigitParams;
      qscale = prm[0];  // the block's score unit
#pragma unroll
      for (int j = 0; j < 4; ++j) dw[j] = prm[1 + j];
      const int kshift = __float_as_int(prm[5]);
      if (kshift > 0) {
        // a mean of more than 2^15 code units: the unit is qs 2^kshift, and
        // the codes are rounded to it (half up; 0 from kshift 8 on)
        const int ksh = min(kshift, 31);
        const int half = 1 << (ksh - 1);
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int x = qf[m][j];
            int y = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) y |= ((((int)(int8_t)(x >> (8 * e))) + half) >> ksh & 0xFF) << (8 * e);
            qf[m][j] = y;
          }
      }
    }
  } else {
#pragma unroll
    for (int m = 0; m < 4; ++m) qf[m] = v4i{0, 0, 0, 0};
  }

  const uint8_t* kbase = p.k8 + (bh * p.nbk + t0) * kTileBytes;
  const uint8_t* vbase = p.v8 + (bh * p.nbk + t0) * kTileBytes;
  const float* ksc = p.ks + bh * p.nbk + t0;

  // Copy tile t into stage `stage`: wave `widx` of `nwaves` copies a
  // contiguous 32/nwaves KiB piece (within the K or the V^T tile).  The LDS
  // destination base lives in M0, and rewriting M0 waits for the previous
  // LDS-DMA to have consumed it, so M0 is set once per 4 KiB and the
  // instruction's immediate offset (added to both addresses) steps by 1 KiB.
  auto copy_tile = [&](int t, int stage, int widx, int nwaves) __attribute__((always_inline)) {
    const int per = 2048 / nwaves;  // 16-byte pieces per wave
    const int c0 = widx * per;      // first piece, wave-uniform
    const int64_t tile = tile_of(t);
    const uint8_t* src = (c0 < 1024 ? kbase + tile * kTileBytes + c0 * 16
                                    : vbase + tile * kTileBytes + (c0 - 1024) * 16) + lane * 16;
    uint8_t* dst = smem + stage * kStage + c0 * 16;
    if constexpr (DS_TABLE) {
      // the first copying wave also brings the tile's Delta-S: lanes 0-31
      // the first query block's 128 values, lanes 32-63 the second's
      if (widx == 0) {
        const int qb = min(2 * mtile + (lane >> 5), p.nbq - 1);
        const float* dsrc = p.ds + ((bh * p.nbq + qb) * (int64_t)p.nbk + t0 + tile) * 128 + (lane & 31) * 4;
        copy_to_lds_off<0>(reinterpret_cast<const uint8_t*>(dsrc), smem + stage * kStage + 2 * kTileBytes);
      }
    }
    for (int i = 0; i < per / 256; ++i) {
      copy_to_lds_off<0>(src + i * 4096, dst + i * 4096);
      copy_to_lds_off<1024>(src + i * 4096, dst + i * 4096);
      copy_to_lds_off<2048>(src + i * 4096, dst + i * 4096);
      copy_to_lds_off<3072>(src + i * 4096, dst + i * 4096);
    }
  };

  float m_run = -__builtin_inff(), l_run = 0.0f;
  v16f O[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) O[db][r] = 0.0f;
  v16i S[4];
  uint32_t P[2][8];
  float c_cur = 0.0f;       // dequant scale of the tile whose S is held
  bool masked_cur = false;  // block-sparse: that tile is masked for this group
  bool pv_skip = false;     // block-sparse: the P registers belong to a masked tile
  int dstage_cur = 0;       // Q smoothing: the LDS stage holding that tile's Delta-S
  // The K block scales are read through the constant address space, which
  // makes these uniform loads scalar (s_load, counted by lgkmcnt).  A vector
  // load here would be followed by a vmcnt wait that also waits for the
  // LDS-DMA of the next tile issued in the same block.
  const __attribute__((address_space(4))) float* ksc4 =
      (const __attribute__((address_space(4))) float*)(ksc);

  // ---- INT8 Q smoothing: Delta-S of tile u (in LDS stage `stage`) for this
  // group's query block, keys 32 kb + [0, 32) with kb = w % 4; each of the
  // group's four waves forms a quarter.  D[r][key] = sum_d a_r[d]
  // kcode[key][d] on the INT8 MFMA, the digit rows as A (lanes 0-3 of each
  // half: rows 0-3, channels 64 hh + 16 m + [0, 16) for MFMA m; the other
  // lanes read zeros) and the keys' codes as B, so lanes 0-31 hold the four
  // digit sums of key 32 kb + lane in registers 0-3.  Their sum
  // sum_r 2^(E - 7r) D_r is formed in FP32, rounded to the unit
  // (|Delta-S| < 2^29) and written to the group's buffer of tile parity
  // u % 2 (the stage count is even, so that is stage % 2).
  // ds_digits reads the digit rows (once per sweep), ds_load the keys'
  // codes, ds_mfma runs the MFMAs, ds_store the sum and the write.
  auto ds_load = [&](int stage, v4i (&kk)[4]) __attribute__((always_inline)) {
    const int row = (w & 3) * 32 + l32;
    const uint8_t* Ks = smem + stage * kStage + row * 128;
#pragma unroll
    for (int m = 0; m < 4; ++m) kk[m] = *reinterpret_cast<const v4i*>(Ks + ((((4 * hh + m) ^ swz(row)) & 7) << 4));
  };
  auto ds_digits = [&](v4i (&dg)[4]) __attribute__((always_inline)) {
    const uint8_t* dgl = smem + kDigOff + (isA ? 0 : 1024) + (l32 < 4 ? l32 * 128 + 64 * hh : 512);
#pragma unroll
    for (int m = 0; m < 4; ++m) dg[m] = *reinterpret_cast<const v4i*>(dgl + 16 * m);
  };
  auto ds_mfma = [&](const v4i (&kk)[4], const v4i (&dg)[4]) __attribute__((always_inline)) -> v16i {
    v16i D = __builtin_amdgcn_mfma_i32_32x32x32_i8(dg[0], kk[0], v16i{}, 0, 0, 0);
#pragma unroll
    for (int m = 1; m < 4; ++m) D = __builtin_amdgcn_mfma_i32_32x32x32_i8(dg[m], kk[m], D, 0, 0, 0);
    return D;
  };
  auto ds_store = [&](int stage, const v16i& D) __attribute__((always_inline)) {
    if (hh == 0) {
      const float f = __builtin_fmaf((float)D[0], dw[0],
                                     __builtin_fmaf((float)D[1], dw[1],
                                                    __builtin_fmaf((float)D[2], dw[2], (float)D[3] * dw[3])));
      reinterpret_cast<int*>(smem + kDsOff + (isA ? 0 : 1024) + (stage & 1) * 512)[(w & 3) * 32 + l32] =
          (int)__builtin_rintf(f);
    }
  };

  // ---- M(t): PV of tile t-1, then S of tile t
  // kst = t % NS, the LDS stage of tile t.  The steady-state loop passes it
  // as a literal, so every LDS address is a lane constant plus an immediate.
  // mask_rem < 128 (the partial last tile only): keys at or past mask_rem
  // get the bits of -inf (FP8 Q/K) or the integer minimum (INT8), which the
  // softmax of that tile turns into p = 0.  The MFMA-issuing wave waits for
  // these S values here, once per sweep.
  // mask_all (block-sparse): this wave group's query block does not attend
  // tile t.  The group skips the tile's score MFMAs, its V phase and its PV
  // MFMAs (wave-uniform branches): the row maximum, the row sum and O stay
  // as they are.
  auto mblock = [&](int t, bool do_pv, bool do_s, int kst, int mask_rem,
                    bool mask_all) __attribute__((always_inline)) {
    // the MFMA-issuing wave of the SIMD gets issue priority over its partner
    __builtin_amdgcn_s_setprio(2);
    // tile t+PD comes in halves: group A's waves copy its K tile here, group
    // B's its V^T tile one slot later (first read two slots after that),
    // 4 KiB per wave, so that each wave writes M0 once per tile
    if (t >= 1 && t + PD < nbk) copy_tile(t + PD, (kst + PD) % NS, w, 8);
    // INT8 Q smoothing: the reads of the operands for the next tile's
    // Delta-S go ahead of the P.V MFMAs, which hide their latency
    v4i dsk[4];
    v16i dsd;
    const bool ds_more = DS_MFMA && do_s && t + 1 < nbk;
    if constexpr (DS_MFMA) {
      if (ds_more) ds_load((kst + 1) % NS, dsk);
    }
    if (do_pv && !(SPARSE && pv_skip)) {
      const uint8_t* Vs = smem + ((kst + NS - 1) % NS) * kStage + kTileBytes;  // stage of t-1
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const v8i Bp = {(int)P[g][0], (int)P[g][1], (int)P[g][2], (int)P[g][3],
                        (int)P[g][4], (int)P[g][5], (int)P[g][6], (int)P[g][7]};
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const int d = db * 32 + l32;
          const uint8_t* vrow = Vs + d * 128;
          const int ch0 = 4 * g + 2 * hh;
          const v4i lo = *reinterpret_cast<const v4i*>(vrow + (((ch0 ^ swz(d)) & 7) << 4));
          const v4i hi = *reinterpret_cast<const v4i*>(vrow + ((((ch0 + 1) ^ swz(d)) & 7) << 4));
          const v8i A = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          O[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, Bp, O[db], 0, 0, 0, 127, 0, 127);
        }
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int i = 0; i < 7; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    if constexpr (SPARSE) {
      if (do_s) masked_cur = mask_all;
    }
    // INT8 Q smoothing: the P.V MFMAs stay ahead of the K operand reads, so
    // that the V operands and the K operands are never live together (the
    // empty asm uses O, and no memory access crosses it)
    if constexpr (DS_MFMA) {
#pragma unroll
      for (int db = 0; db < 4; ++db) asm volatile("" ::"v"(O[db]) : "memory");
      __builtin_amdgcn_sched_barrier(0);
      // the next tile's Delta-S MFMAs (summed and stored after the score
      // MFMAs, off their path), then this tile's Delta-S, the score
      // accumulators' initial values (register 4a + b of block kb is key
      // 32 kb + 8a + 4 hh + b; S is free here)
      if (ds_more) dsd = ds_mfma(dsk, dgr);
      if (do_s) {
        const int* dsr = reinterpret_cast<const int*>(smem + kDsOff + (isA ? 0 : 1024) + (kst & 1) * 512);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const v4i d4 = *reinterpret_cast<const v4i*>(dsr + 32 * kb + 8 * a + 4 * hh);
#pragma unroll
            for (int b2 = 0; b2 < 4; ++b2) S[kb][4 * a + b2] = d4[b2];
          }
      }
    }
    if (do_s && !(SPARSE && mask_all)) {
      const uint8_t* Ks = smem + kst * kStage;
      v4i kf[4][4];
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const int row = kb * 32 + l32;
          kf[kb][m] = *reinterpret_cast<const v4i*>(Ks + row * 128 + ((((4 * hh + m) ^ swz(row)) & 7) << 4));
        }
      // m-outer: the four accumulation chains (one per key block) interleave,
      // so no MFMA waits on the result of the one just issued
      if constexpr (FP8QK) {
        // channels 64 hh + 32 c + [0, 32) feed the MFMA of half c
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            const v4i a0 = kf[kb][2 * c], a1 = kf[kb][2 * c + 1];
            const v4i b0 = qf[2 * c], b1 = qf[2 * c + 1];
            const v8i A = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            const v8i Bq = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
            const v16f acc = c == 0 ? v16f{} : __builtin_bit_cast(v16f, S[kb]);
            S[kb] = __builtin_bit_cast(
                v16i, __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, Bq, acc, 0, 0, 0, 127, 0, 127));
          }
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int i = 0; i < 6; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      } else if constexpr (DS_MFMA) {
        // the scores, accumulated onto Delta-S (read at the start of the phase)
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) S[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[kb][m], qf[m], S[kb], 0, 0, 0);
        if (ds_more) ds_store((kst + 1) % NS, dsd);
      } else {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) S[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[kb][0], qf[0], v16i{}, 0, 0, 0);
#pragma unroll
        for (int m = 1; m < 4; ++m)
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) S[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[kb][m], qf[m], S[kb], 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int i = 0; i < 12; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      }
      // (Q smoothing: a block with qs = 0 has all-zero codes; its scores are
      // the Delta-S table's values, held in units of 2^-20 * ks)
      c_cur = (DS_TABLE && qscale == 0.0f ? 0x1p-20f : qscale) * ksc4[tile_of(t)] * p.sl2e;
      if constexpr (DS_TABLE) dstage_cur = kst;
      if (mask_rem < 128) {
        // the first masked key offset of this lane half; the empty asm before
        // each comparison keeps the 64 lane masks from all being computed up
        // front and held in SGPRs
        int rl = mask_rem - 4 * hh;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            asm volatile("" : "+v"(rl));
            if (kb * 32 + 8 * (r >> 2) + (r & 3) >= rl) S[kb][r] = FP8QK ? kNegInfBits : kIntMin;
          }
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // INT8 score as a float: the exact conversion of the accumulator; in the
  // masked last tile the integer minimum stands for -inf
  auto score_f = [&](int s, bool masked) __attribute__((always_inline)) -> float {
    if constexpr (FP8QK) return __int_as_float(s);
    else return masked && s == kIntMin ? -__builtin_inff() : (float)s;
  };

  // ---- V(t): online softmax of S -> P, conditional rescale of O
  // first: the sweep's first tile (m = -inf, O = 0 and l = 0 before it), where
  // the rescale would multiply zeros by exp2(-inf); the block-sparse instance
  // keeps it, since its first attended tile depends on the table.
  // masked: the tile holds keys past Nkv (the sweep's last tile only).
  auto vblock = [&](bool first, bool masked) __attribute__((always_inline)) {
    if constexpr (SPARSE) {
      pv_skip = masked_cur;
      if (masked_cur) return;
    }
    // c = 0 (an all-zero Q or K block: every score of the tile is 0) would
    // turn masked keys' -inf into NaN; the smallest normal float gives the
    // same exponent arguments for the valid keys (its products stay far
    // below their rounding unit) and keeps -inf at -inf.
    const float c = c_cur == 0.0f ? 1.17549435e-38f : c_cur;
    float mt;
    if constexpr (DS_TABLE) {
      // add Delta-S (in the units of S: the table holds (qmean . kcode) / qs)
      // of this group's query block to every score, written back over S,
      // then the row maximum on floats; masked keys are -inf.  The sum is
      // rounded once, at the score's own magnitude.
      const float* dsl = reinterpret_cast<const float*>(smem + dstage_cur * kStage + 2 * kTileBytes) +
                         (isA ? 0 : 128) + 4 * hh;
      float mx = -__builtin_inff();
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const float4 d4 = *reinterpret_cast<const float4*>(dsl + 32 * kb + 8 * a);
          const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int b2 = 0; b2 < 4; ++b2) {
            const int r = 4 * a + b2;
            const float tt = score_f(S[kb][r], masked) + dv[b2];
            S[kb][r] = __float_as_int(tt);
            mx = fmaxf(mx, tt);
          }
        }
      mx = fmaxf(mx, other_half_f(mx));
      mt = mx * c;
    } else if constexpr (FP8QK) {
      // FP32 scores (unscaled); masked keys are -inf
      float mx = -__builtin_inff();
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, __int_as_float(S[kb][r]));
      mx = fmaxf(mx, other_half_f(mx));
      mt = mx * c;
    } else {
      int mx = kIntMin;  // masked keys hold the minimum; every tile has a valid key
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = max(mx, (int)S[kb][r]);
      mx = max(mx, other_half_i(mx));
      mt = (float)mx * c;
    }
    const float mnew = fmaxf(m_run, mt);
    if (!(first && !SPARSE) && __any(mnew > m_run)) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - mnew);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) O[db][r] *= alpha;
    }
    m_run = mnew;
    // exponent argument fma(s, c, nb) = (score - m) log2 e + log2 448 with
    // nb = log2 448 - m, rounded once, s the exact float value of the INT8
    // accumulator (one conversion per score).  Reading the accumulators as
    // floats through a bias 1.5 * 2^23 in their initial value, and folding
    // that bias into nb, would save the conversion but round nb at the
    // magnitude of 1.5 * 2^23 c: a per-tile shift of the reference point that
    // moves P's E4M3 rounding and reweights a row's tiles, by more than the
    // accuracy bar at sharp softmax scales.
    const float nb = kLog2_448 - mnew;
    float ls[4];
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int kb = 2 * g + (j >> 2);
        const int r0 = 4 * (j & 3);
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float sf = DS_TABLE ? __int_as_float(S[kb][r0 + i]) : score_f(S[kb][r0 + i], masked);
          pv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sf, c, nb));
          // the first term starts the sum (p >= 0, so 0 + p == p)
          ls[i] = (g == 0 && j == 0) ? pv[i] : ls[i] + pv[i];
        }
        // the first conversion writes the low half only: start from the
        // register's old contents instead of materialising a zero
        int wd = __builtin_amdgcn_cvt_pk_fp8_f32(pv[0], pv[1], (int)P[g][j], false);
        wd = __builtin_amdgcn_cvt_pk_fp8_f32(pv[2], pv[3], wd, true);
        P[g][j] = (uint32_t)wd;
      }
    l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);
    // The results leave the phase here: without these uses the compiler is
    // free to sink the exponentials past the next barrier into the partner
    // group's phase, which would undo the MFMA / VALU alternation.
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int j = 0; j < 8; ++j) asm volatile("" ::"v"(P[g][j]));
    asm volatile("" ::"v"(l_run));
  };

  // The barrier builtin does not order memory for the compiler: the empty
  // asm with a memory clobber on each side keeps every LDS access (the
  // tile reads, the epilogue's staging) on its side of the barrier.  It
  // adds no instruction and no wait.
  auto barrier = [] {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  auto wait_loads = [] { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int j = 0; j < 8; ++j) P[g][j] = 0u;

  // INT8 Q smoothing: the first wave of each group copies its block's four
  // digit rows (512 bytes; zeros past the last block) into the group's LDS
  // area, followed by 64 zero bytes, the operand of the A rows 4-31
  if constexpr (DS_MFMA) {
    if ((w & 3) == 0) {
      uint8_t* dst = smem + kDigOff + (isA ? 0 : 1024);
      uint2 v = make_uint2(0u, 0u);
      if (q0 < p.nbq * 128) v = reinterpret_cast<const uint2*>(p.dg + (bh * p.nbq + qblk) * kDigitBytes)[lane];
      reinterpret_cast<uint2*>(dst)[lane] = v;
      if (lane < 8) reinterpret_cast<uint2*>(dst + 512)[lane] = make_uint2(0u, 0u);
    }
  }

  // prologue: tiles 0 .. PD into their stages, all waves copying (INT8 Q
  // smoothing: then the first tile's Delta-S)
  copy_tile(0, 0, w, 8);
  if (nbk > 1) copy_tile(1, 1, w, 8);
  if (PD > 1 && nbk > 2) copy_tile(2, 2, w, 8);
  wait_loads();
  __syncthreads();
  if constexpr (DS_MFMA) {
    v4i kk[4];
    ds_digits(dgr);
    ds_load(0, kk);
    ds_store(0, ds_mfma(kk, dgr));
    __syncthreads();
  }

  if (!isA) barrier();  // group B lags one slot
  const int last = nbk - 1;
  // keys in the last tile: the head's partial tail only in the last split
  // (block-sparse: when the head's last tile is listed, it is listed last)
  int rem = t0 + nbk == p.nbk ? p.Nkv - (p.nbk - 1) * 128 : 128;
  if constexpr (SPARSE) rem = tile_of(last) == p.nbk - 1 ? p.Nkv - (p.nbk - 1) * 128 : 128;
  auto step = [&](int t, bool do_pv, int kst) __attribute__((always_inline)) {
    mblock(t, do_pv, true, kst, 128, SPARSE && !group_attends(t));
    barrier();
    vblock(!do_pv, false);
    wait_loads();
    barrier();
  };
  int t = 0;
  if (last > 0) {
    step(0, false, 0);
    t = 1;
  }
  if constexpr (NS == 4) {
    for (; t + 4 <= last; t += 4) {
      step(t, true, 1);
      step(t + 1, true, 2);
      step(t + 2, true, 3);
      step(t + 3, true, 0);
    }
  } else {
    for (; t + 3 <= last; t += 3) {
      step(t, true, 1);
      step(t + 1, true, 2);
      step(t + 2, true, 0);
    }
  }
  for (; t < last; ++t) step(t, true, t % NS);
  mblock(last, last > 0, true, last % NS, rem, SPARSE && !group_attends(last));
  barrier();
  vblock(last == 0, rem < 128);
  wait_loads();
  barrier();
  mblock(nbk, true, false, nbk % NS, 128, false);
  if (isA) barrier();

  // ---- epilogue: O = acc * vs / l448 -> BF16 (or FP32 partials of a split)
  pin_accumulators(O);
  const float* vsc = p.vs + bh * 128;
  const float lt = l_run + other_half_f(l_run);
  const int q = q0 + l32;
  // log-sum-exp of the row over this workgroup's keys, natural log:
  // ln 2 * (m + log2(l448 / 448)) for the smoothed scores; and (when the
  // caller asked for the LSE) the logit shift the K smoothing removed,
  // softmax_scale * qs * sum_d qc_d kmean_d, from the Q codes this lane
  // holds (channels 64 hh + [0, 64); with INT8 Q smoothing qs is the
  // block's unit and the codes those the scores used).  Split partials
  // carry no shift, so the merged output does not depend on whether the
  // LSE is asked for.
  float lse = 0.0f, shift = 0.0f;
  if (p.lse != nullptr || p.splits > 1) lse = kLn2 * (m_run + log2f(lt) - kLog2_448);
  if (p.lse != nullptr) {
    const float* kmr = p.km + bh * 128 + 64 * hh;
    float acc = 0.0f;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
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
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = __builtin_fmaf(qc[e], kmr[16 * m + 4 * j + e], acc);
      }
    float accm = 0.0f;
    if constexpr (QSMOOTH) {
      // plus the Q block mean against the K mean
      const float* qmr = p.qm + (bh * p.nbq + min(qblk, p.nbq - 1)) * 128 + 64 * hh;
#pragma unroll
      for (int d = 0; d < 64; ++d) accm = __builtin_fmaf(qmr[d], kmr[d], accm);
    }
    acc += other_half_f(acc);
    accm += other_half_f(accm);
    shift = p.scale * (qscale * acc + accm);
  }
  // (block-sparse: a row whose query block attends none of the listed
  // tiles has l = 0, O = 0 and lse = -inf)
  const float inv = SPARSE && lt == 0.0f ? 0.0f : 1.0f / lt;
  if (p.splits == 1) {
    // BF16 rows through 4 KiB of LDS per wave, 64 channels at a time: each
    // lane holds 4-channel pieces of its row, so direct stores would write
    // 8 bytes into each of 32 rows per instruction; staged, every global
    // store writes whole 128-byte lines (8 lanes per row).  The area is the
    // stage of the never-loaded tile nbk, whose last reader (tile nbk-NS's
    // PV) is two barriers back or more.  Chunks are XOR-swizzled by (row >> 1) & 7
    // so the piece writes of 32 rows spread over the banks.  LDS operations
    // of one wave run in order, so the second half's writes land after the
    // first half's reads.
    uint8_t* obuf = smem + (nbk % NS) * kStage + w * 4096;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      // (keeps the compiler from hoisting the second half's scale loads
      // above the first half: fewer registers live at once)
      asm volatile("" ::: "memory");
#pragma unroll
      for (int db2 = 0; db2 < 2; ++db2)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int db = 2 * half + db2;
          const int d0 = 32 * db + 8 * a + 4 * hh;
          const float4 sv = *reinterpret_cast<const float4*>(vsc + d0);
          const float o0 = O[db][4 * a + 0] * sv.x * inv;
          const float o1 = O[db][4 * a + 1] * sv.y * inv;
          const float o2 = O[db][4 * a + 2] * sv.z * inv;
          const float o3 = O[db][4 * a + 3] * sv.w * inv;
          const int c = 4 * db2 + a;
          *reinterpret_cast<uint2*>(obuf + l32 * 128 + (((c ^ swz(l32)) & 7) << 4) + 8 * hh) =
              make_uint2(bf16_rne(o0) | (bf16_rne(o1) << 16), bf16_rne(o2) | (bf16_rne(o3) << 16));
        }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 8 * i + (lane >> 3), c = lane & 7;
        const uint4 val = *reinterpret_cast<const uint4*>(obuf + r * 128 + (((c ^ swz(r)) & 7) << 4));
        const int qr = q0 + r;
        if (qr < p.Nq)
          *reinterpret_cast<uint4*>(p.out + b * p.os0 + (int64_t)qr * p.os1 + h * p.os2 + 64 * half + 8 * c) = val;
      }
    }
    if (p.lse != nullptr && hh == 0 && q < p.Nq) p.lse[bh * p.Nq + q] = lse + shift;
  } else if (q < p.Nq) {
    const int64_t row = ((int64_t)split * p.BH + bh) * p.Nq + q;
    float* orow = p.opart + row * 128;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d0 = 32 * db + 8 * a + 4 * hh;
        const float4 sv = *reinterpret_cast<const float4*>(vsc + d0);
        *reinterpret_cast<float4*>(orow + d0) =
            make_float4(O[db][4 * a + 0] * sv.x * inv, O[db][4 * a + 1] * sv.y * inv,
                        O[db][4 * a + 2] * sv.z * inv, O[db][4 * a + 3] * sv.w * inv);
      }
    if (hh == 0) p.lpart[row] = lse;
    // the merge kernel adds the partials' lse to the shift left here
    if (p.lse != nullptr && split == 0 && hh == 0) p.lse[bh * p.Nq + q] = shift;
  }
}

// Merge of split partials: row r = bh * Nq + q gets
//   lse = ln sum_s exp(lse_s),  O = sum_s exp(lse_s - lse) O_s  -> BF16,
// the log-sum-exp rule; the LSE output (if any) already holds the row's
// smoothing shift, written by the attention kernel, and gets lse added.
// 32 threads per row, 4 channels each.
struct CombP {
  const float* opart;
  const float* lpart;
  uint16_t* out;
  float* lse;
  int64_t os0, os1, os2;
  int64_t rows;  // B*H*Nq
  int H, Nq, splits;
};

__global__ __launch_bounds__(256) void k_combine(CombP p) {
  const int64_t r = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
  if (r >= p.rows) return;
  const int c0 = (threadIdx.x & 31) * 4;
  float mx = -__builtin_inff();
  for (int s = 0; s < p.splits; ++s) mx = fmaxf(mx, p.lpart[s * p.rows + r]);
  float wsum = 0.0f;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int s = 0; s < p.splits; ++s) {
    const float w = __builtin_amdgcn_exp2f((p.lpart[s * p.rows + r] - mx) * kLog2e);
    const float4 o = *reinterpret_cast<const float4*>(p.opart + (s * p.rows + r) * 128 + c0);
    wsum += w;
    acc.x = __builtin_fmaf(w, o.x, acc.x);
    acc.y = __builtin_fmaf(w, o.y, acc.y);
    acc.z = __builtin_fmaf(w, o.z, acc.z);
    acc.w = __builtin_fmaf(w, o.w, acc.w);
  }
  const float inv = 1.0f / wsum;
  const int64_t bh = r / p.Nq, q = r % p.Nq;
  uint16_t* orow = p.out + (bh / p.H) * p.os0 + q * p.os1 + (bh % p.H) * p.os2 + c0;
  *reinterpret_cast<uint2*>(orow) =
      make_uint2(bf16_rne(acc.x * inv) | (bf16_rne(acc.y * inv) << 16),
                 bf16_rne(acc.z * inv) | (bf16_rne(acc.w * inv) << 16));
  if (p.lse != nullptr && c0 == 0) p.lse[r] += mx + kLn2 * log2f(wsum);
}

// Block mask [B][H][nbq][nbk] (nonzero = attend) -> per query tile of 256
// rows (query blocks 2m, 2m+1) the ascending list of key tiles either block
// attends, each entry the tile index | bit 30 (block 2m attends) | bit 31
// (block 2m+1 attends), and the list's length.  One wave per query tile: 64
// key tiles per step, compacted in order through a ballot.
struct LutP {
  const uint8_t* mask;
  int32_t* counts;
  uint32_t* entries;
  int64_t G;  // B*H*mt
  int nbq, nbk, mt;
};

__global__ __launch_bounds__(256) void k_block_lut(LutP p) {
  const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (g >= p.G) return;
  const int lane = threadIdx.x & 63;
  const int64_t bh = g / p.mt;
  const int qb0 = 2 * (int)(g % p.mt);
  const bool two = qb0 + 1 < p.nbq;
  const uint8_t* m0 = p.mask + (bh * p.nbq + qb0) * p.nbk;
  const uint8_t* m1 = m0 + p.nbk;
  uint32_t* out = p.entries + g * p.nbk;
  int count = 0;
  for (int k0 = 0; k0 < p.nbk; k0 += 64) {
    const int kb = k0 + lane;
    const bool a0 = kb < p.nbk && m0[kb] != 0;
    const bool a1 = kb < p.nbk && two && m1[kb] != 0;
    const uint64_t any = __ballot(a0 || a1);
    const int pos = count + __popcll(any & ((1ull << lane) - 1ull));
    if (a0 || a1) out[pos] = (uint32_t)kb | (a0 ? 1u << 30 : 0u) | (a1 ? 1u << 31 : 0u);
    count += __popcll(any);
  }
  if (lane == 0) p.counts[g] = count;
}

template <bool FP8QK, bool SPARSE, bool QSMOOTH>
hipError_t launch_pp(const AttnArgs& a, hipStream_t stream) {
  const Layout& L = a.L;
  constexpr int BM = 256;
  // three K/V stages (E4M3 Q smoothing: each with its Delta-S rows); INT8 Q
  // smoothing: four, then 1 KiB of Delta-S and 1 KiB of digit rows per group
  constexpr int kLds = QSMOOTH && !FP8QK ? 4 * kStageBytes + 2048 + 2048 : 3 * (kStageBytes + (QSMOOTH ? 1024 : 0));
  // Raising the dynamic LDS limit is per function and device, once each.
  // The flags are atomics: threads that race here may both set the
  // attribute (the same value, harmless), with no unsynchronised access.
  constexpr int kMaxDev = 64;
  static std::atomic<bool> attr_set[kMaxDev];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev || !attr_set[dev].load(std::memory_order_acquire)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_pp_kernel<FP8QK, SPARSE, QSMOOTH>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kMaxDev) attr_set[dev].store(true, std::memory_order_release);
  }
  AttnP p;
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
  p.splits = a.splits;
  p.tps = a.tps;
  p.opart = a.splits > 1 ? reinterpret_cast<float*>(a.workspace) : nullptr;
  p.lpart = a.splits > 1 ? reinterpret_cast<float*>(a.workspace + split_opart_bytes(a.splits, p.BH, L.Nq))
                         : nullptr;
  p.H = (int)L.H;
  p.Nq = (int)L.Nq;
  p.Nkv = (int)L.Nkv;
  p.nbq = (int)L.nbq;
  p.nbk = (int)L.nbk;
  p.mt = (int)((L.Nq + BM - 1) / BM);
  p.G = p.BH * p.splits * p.mt;
  p.scale = a.softmax_scale;
  p.sl2e = a.softmax_scale * kLog2e;
  const int64_t G8 = (p.G + 7) / 8 * 8;
  p.lut_counts = a.lut_counts;
  p.lut_entries = a.lut_entries;
  p.ds = QSMOOTH && FP8QK ? reinterpret_cast<const float*>(a.packed + L.off_ds) : nullptr;
  p.dg = QSMOOTH && !FP8QK ? reinterpret_cast<const int8_t*>(a.packed + L.off_dg) : nullptr;
  p.dp = QSMOOTH && !FP8QK ? reinterpret_cast<const float*>(a.packed + L.off_dp) : nullptr;
  p.qm = QSMOOTH ? reinterpret_cast<const float*>(a.packed + L.off_qm) : nullptr;
  hipLaunchKernelGGL((attn_pp_kernel<FP8QK, SPARSE, QSMOOTH>), dim3((unsigned)G8), dim3(512), kLds, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  return launch_combine(p.opart, p.lpart, a, stream);
}

}  // namespace

hipError_t launch_combine(const float* opart, const float* lpart, const AttnArgs& a, hipStream_t stream) {
  const int64_t BH = a.L.B * a.L.H;
  CombP c{opart, lpart, a.out, a.lse, a.o_str[0], a.o_str[1], a.o_str[2], BH * a.L.Nq, (int)a.L.H,
          (int)a.L.Nq, a.splits};
  hipLaunchKernelGGL(k_combine, dim3((unsigned)((c.rows + 7) / 8)), dim3(256), 0, stream, c);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, bool cross, hipStream_t stream) {
  (void)cross;
  if (a.lut_counts != nullptr)
    return a.fp8qk ? launch_pp<true, true, false>(a, stream) : launch_pp<false, true, false>(a, stream);
  if (a.L.qsmooth)
    return a.fp8qk ? launch_pp<true, false, true>(a, stream) : launch_pp<false, false, true>(a, stream);
  if (short_kv_applies(a)) return launch_attention_short(a, stream);
  return a.fp8qk ? launch_pp<true, false, false>(a, stream) : launch_pp<false, false, false>(a, stream);
}

hipError_t launch_block_lut(const uint8_t* mask, const Layout& L, uint8_t* lut, hipStream_t stream) {
  LutP p;
  p.mask = mask;
  p.mt = (int)((L.Nq + 255) / 256);
  p.G = L.B * L.H * p.mt;
  p.nbq = (int)L.nbq;
  p.nbk = (int)L.nbk;
  p.counts = reinterpret_cast<int32_t*>(lut);
  p.entries = reinterpret_cast<uint32_t*>(lut + lut_counts_bytes(p.G));
  hipLaunchKernelGGL(k_block_lut, dim3((unsigned)((p.G + 3) / 4)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sattn
