// layout.h -- packed-buffer layout shared by the host API and the kernels.
//
// The preprocessing step writes Q/K/V codes in the order the attention kernel
// consumes them (the MHA v4 page, "Technical Details": preprocessing kept
// separate from attention, with specialized packed layouts behind a size
// query; its import listing shows K written in LDS order and V stored
// column-major).  All sections are 256-byte aligned:
//
//   q8   [B][H][nbq] tiles of 128 tokens x 128 channels int8, row-major
//        (token, channel); rows past Nq are zero.  Loaded straight into
//        registers as the B operand of the K.Q^T MFMA.
//   k8   [B][H][nbk] tiles, row-major (key, channel) with the 16-byte chunk
//        index XOR-ed with ((key >> 1) & 7).  gfx950's LDS serves a 16-byte
//        read for 16 lanes per cycle across 64 banks (256 bytes); sixteen
//        lanes reading the same logical chunk of sixteen consecutive keys
//        then hit sixteen different 16-byte bank groups (row r starts at
//        bank group 8(r & 1)).  Rows past Nkv are zero.
//   v8   [B][H][nbk] tiles of V^T: row = channel d (128 rows), 128 key
//        columns.  Inside each group of 64 keys the columns follow the
//        k-index order of the FP8 MFMA B operand as the K.Q^T accumulator
//        leaves P in registers (see v_col below), so P never moves between
//        lanes; the 16-byte chunks are XOR-swizzled with ((d >> 1) & 7).
//        Columns of keys past Nkv are zero.
//   q_scale [B][H][nbq], k_scale [B][H][nbk], v_scale [B][H][128],
//   k_mean  [B][H][128]  (FP32)
//   with Q smoothing only:
//   q_mean  [B][H][nbq][128]  FP32 block means of Q
//   d_s     [B][H][nbq][nbk * 128]  FP32 Delta-S: for query block i and key
//           j, (q_mean[i] . kcode[j]) / u_i with u_i = qs_i (2^-20 if qs_i = 0),
//           in the units of the Q.K^T accumulator of block i; entries of keys
//           past Nkv are zero.
//
// Workspace: k_part [B][H][nbk][128] FP32 block sums of K and v_part
// [B][H][nbk][128] FP32 block maxima of |V|.
#pragma once
#include <stddef.h>
#include <stdint.h>

#ifdef __HIPCC__
#define SATTN_HD __host__ __device__
#else
#define SATTN_HD
#endif

namespace sattn {

constexpr int kD = 128;
constexpr int kBlk = 128;
constexpr int64_t kTileBytes = 128 * 128;

SATTN_HD inline int64_t nblocks(int64_t n) { return (n + kBlk - 1) / kBlk; }
SATTN_HD inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Q smoothing, INT8 codes: per Q block, four rows of int8 digits of the
// block mean over its score unit (kDigitBytes), and the unit, the digits'
// four weights and the code shift (kDigitParams floats).
constexpr int64_t kDigitBytes = 4 * 128;
constexpr int64_t kDigitParams = 8;

struct Layout {
  int64_t B, H, Nq, Nkv, nbq, nbk;
  bool qsmooth, fp8qk;
  size_t off_q8, off_k8, off_v8, off_qs, off_ks, off_vs, off_km, off_qm, off_ds, off_dg, off_dp, packed_bytes;
  size_t ws_kpart, ws_vpart, workspace_bytes;
};

// Callers validate sizes first (no overflow for N <= 2^24, B*H <= 2^31, and
// for Q smoothing in the FP8 Q/K format the Delta-S section below 2^40
// bytes).  The sections before the Q means do not depend on the format.
inline Layout make_layout(int64_t B, int64_t H, int64_t Nq, int64_t Nkv, bool qsmooth = false,
                          bool fp8qk = false) {
  Layout L;
  L.B = B; L.H = H; L.Nq = Nq; L.Nkv = Nkv;
  L.qsmooth = qsmooth;
  L.fp8qk = fp8qk;
  L.nbq = nblocks(Nq);
  L.nbk = nblocks(Nkv);
  const size_t bh = (size_t)B * (size_t)H;
  size_t o = 0;
  L.off_q8 = o; o = align256(o + bh * (size_t)L.nbq * kTileBytes);
  L.off_k8 = o; o = align256(o + bh * (size_t)L.nbk * kTileBytes);
  L.off_v8 = o; o = align256(o + bh * (size_t)L.nbk * kTileBytes);
  L.off_qs = o; o = align256(o + bh * (size_t)L.nbq * 4);
  L.off_ks = o; o = align256(o + bh * (size_t)L.nbk * 4);
  L.off_vs = o; o = align256(o + bh * kD * 4);
  L.off_km = o; o = align256(o + bh * kD * 4);
  L.off_qm = L.off_ds = L.off_dg = L.off_dp = 0;
  if (qsmooth) {
    L.off_qm = o; o = align256(o + bh * (size_t)L.nbq * kD * 4);
    if (fp8qk) {
      L.off_ds = o; o = align256(o + bh * (size_t)L.nbq * (size_t)L.nbk * kBlk * 4);
    } else {
      L.off_dg = o; o = align256(o + bh * (size_t)L.nbq * kDigitBytes);
      L.off_dp = o; o = align256(o + bh * (size_t)L.nbq * kDigitParams * 4);
    }
  }
  L.packed_bytes = o;
  size_t w = 0;
  L.ws_kpart = w; w = align256(w + bh * (size_t)L.nbk * kD * 4);
  L.ws_vpart = w; w = align256(w + bh * (size_t)L.nbk * kD * 4);
  L.workspace_bytes = w;
  return L;
}

// Byte offset of (token r, channel c) inside a Q tile.
SATTN_HD inline int q_pos(int r, int c) { return r * 128 + c; }

// XOR pattern of the 16-byte chunks of a K or V^T tile row.
SATTN_HD inline int swz(int row) { return (row >> 1) & 7; }

// Byte offset of (key r, channel c) inside a K tile.
SATTN_HD inline int k_pos(int r, int c) { return r * 128 + ((((c >> 4) ^ swz(r)) & 7) << 4) + (c & 15); }

// Column of key j (0..127) inside a V^T tile row.  Within a 64-key group the
// K.Q^T accumulator of the 32x32 INT8 MFMA gives lane half hh the keys
// 8a + 4hh + b of each 32-key block (a = 0..3, b = 0..3); the 32x32x64 FP8
// MFMA takes k-index 32hh + e from lane half hh.  Column 32hh + e therefore
// holds key 32(e/16) + 8((e%16)/4) + 4hh + e%4.
SATTN_HD inline int v_col(int j) {
  const int g = j >> 6, kl = j & 63;
  const int hh = (kl >> 2) & 1;
  const int e = ((kl >> 5) & 1) * 16 + ((kl >> 3) & 3) * 4 + (kl & 3);
  return 64 * g + 32 * hh + e;
}

// Byte offset of (key j, channel d) inside a V^T tile.
SATTN_HD inline int v_pos(int j, int d) {
  const int col = v_col(j);
  return d * 128 + ((((col >> 4) ^ swz(d)) & 7) << 4) + (col & 15);
}

}  // namespace sattn
