// kernels.h -- launchers implemented in the .hip translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace sattn {

struct QuantArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  int64_t q_str[3], k_str[3], v_str[3];  // element strides (batch, seq, head)
  Layout L;
  uint8_t* packed;
  uint8_t* workspace;
  bool fp8qk;  // Q/K as E4M3 with block scale amax/448 instead of INT8 (amax/127)
};

struct AttnArgs {
  const uint8_t* packed;
  Layout L;
  float softmax_scale;
  uint16_t* out;
  int64_t o_str[3];
  bool fp8qk;  // the packed Q/K codes are E4M3
  float* lse;  // [B][H][Nq] natural-log LSE of the logits before smoothing, or null
  int splits;  // key-tile ranges swept by separate workgroups (1: no split)
  int tps;     // key tiles per split
  uint8_t* workspace;  // split partials (splits > 1), split_workspace_bytes() long
  const int32_t* lut_counts;    // block-sparse LUT (null: dense), from launch_block_lut
  const uint32_t* lut_entries;
};

// Block-sparse LUT: per query tile of 256 rows (g = (b*H + h)*mt + m, mt =
// ceil(Nq/256)) an int32 count, then [g][nbk] uint32 entries (key tile |
// bit 30 if query block 2m attends it | bit 31 if block 2m+1 does),
// ascending; each section 256-byte aligned.
inline int64_t lut_counts_bytes(int64_t g) { return align256(g * 4); }
inline int64_t block_lut_bytes(int64_t B, int64_t H, int64_t Nq, int64_t nbk) {
  const int64_t g = B * H * ((Nq + 255) / 256);
  return lut_counts_bytes(g) + align256(g * nbk * 4);
}

// Split-KV workspace: FP32 partial outputs [splits][B*H][Nq][128], then
// their LSE [splits][B*H][Nq], each section 256-byte aligned.
inline int64_t split_opart_bytes(int64_t splits, int64_t bh, int64_t nq) {
  return align256(splits * bh * nq * 128 * 4);
}
inline int64_t split_workspace_bytes(int64_t splits, int64_t bh, int64_t nq) {
  return splits <= 1 ? 0 : split_opart_bytes(splits, bh, nq) + align256(splits * bh * nq * 4);
}

hipError_t launch_quantize(const QuantArgs& a, hipStream_t stream);
// Size and device address (on the current device) of the static workspace
// that sattn_quantize_qkv_noalloc uses instead of a caller's.
constexpr size_t kNoallocWorkspaceBytes = (size_t)16 << 20;
hipError_t noalloc_workspace(uint8_t** out);
hipError_t launch_attention(const AttnArgs& a, bool cross, hipStream_t stream);
// short key sequences (at most four 128-key tiles), many query tiles, no
// split, dense: persistent workgroups with the head's K/V resident in LDS
bool short_kv_applies(const AttnArgs& a);
hipError_t launch_attention_short(const AttnArgs& a, hipStream_t stream);
// merge of split-KV partials (FP32 outputs and LSE) into out and lse
hipError_t launch_combine(const float* opart, const float* lpart, const AttnArgs& a, hipStream_t stream);
hipError_t launch_e4m3_encode(const float* x, uint8_t* out, int64_t n, hipStream_t stream);
hipError_t launch_block_lut(const uint8_t* mask, const Layout& L, uint8_t* lut, hipStream_t stream);

}  // namespace sattn
