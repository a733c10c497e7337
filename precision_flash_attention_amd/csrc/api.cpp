// api.cpp -- the C ABI of libsattn (declared in include/sattn.h): argument
// validation, packed-buffer layout, device check and kernel launches on the
// caller's stream.
//
// As the gfx1201 backend page requires of its backend ("Changes": it raises
// on unsupported devices and on causal, mask, dropout and packed
// multi-sequence inputs "instead of computing something else"), every call
// validates all of its arguments before touching the device and returns an
// error status, never a different computation.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <cmath>

#include "../../include/sattn.h"
#include "kernels.h"
#include "layout.h"

using sattn::Layout;

namespace {

// B*H*N*128 BF16 elements must stay below 2^40 bytes: far above any device
// memory, and keeps every grid and index computation inside 32/64-bit ranges.
constexpr int64_t kMaxElems = (int64_t)1 << 39;

sattn_status check_dims(int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t D) {
  if (B <= 0 || H <= 0 || Nq <= 0 || Nkv <= 0 || D <= 0) return SATTN_ERR_INVALID_ARGUMENT;
  if (D != SATTN_HEAD_DIM) return SATTN_ERR_UNSUPPORTED;
  if (Nq > SATTN_MAX_SEQ || Nkv > SATTN_MAX_SEQ) return SATTN_ERR_UNSUPPORTED;
  if (B > kMaxElems || H > kMaxElems) return SATTN_ERR_INVALID_ARGUMENT;
  const int64_t bh = B * H;  // both <= 2^39 but the product may overflow
  if (B != 0 && bh / B != H) return SATTN_ERR_INVALID_ARGUMENT;
  const int64_t nmax = Nq > Nkv ? Nq : Nkv;
  const int64_t rows = (sattn::nblocks(nmax) * SATTN_BLOCK);
  if (bh > kMaxElems / (rows * SATTN_HEAD_DIM)) return SATTN_ERR_INVALID_ARGUMENT;
  if (bh * sattn::nblocks(nmax) > SATTN_MAX_BLOCKS) return SATTN_ERR_UNSUPPORTED;
  return SATTN_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// strides: NULL = contiguous BSHD; otherwise non-negative multiples of 8.
sattn_status get_strides(const int64_t* s, int64_t N, int64_t H, int64_t out[3]) {
  if (s == nullptr) {
    out[0] = N * H * SATTN_HEAD_DIM;
    out[1] = H * SATTN_HEAD_DIM;
    out[2] = SATTN_HEAD_DIM;
    return SATTN_OK;
  }
  for (int i = 0; i < 3; ++i) {
    if (s[i] < 0 || (s[i] % 8) != 0 || s[i] > kMaxElems) return SATTN_ERR_INVALID_ARGUMENT;
    out[i] = s[i];
  }
  return SATTN_OK;
}

// Per-device result of the gfx950 check: 0 unknown, 1 ok, 2 not gfx950.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch[kMaxDevices];

sattn_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return SATTN_ERR_DEVICE;
  const char* forced = getenv("SATTN_TEST_FORCE_ARCH");  // error-path tests only
  if (forced != nullptr) return strncmp(forced, "gfx950", 6) == 0 ? SATTN_OK : SATTN_ERR_DEVICE;
  if (dev >= kMaxDevices) return SATTN_ERR_DEVICE;
  int st = g_arch[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return SATTN_ERR_DEVICE;
    st = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch[dev].store(st, std::memory_order_release);
  }
  return st == 1 ? SATTN_OK : SATTN_ERR_DEVICE;
}

sattn_status launch_status(hipError_t e) { return e == hipSuccess ? SATTN_OK : SATTN_ERR_LAUNCH; }

// qk_format: a sattn_qk_format, optionally OR-ed with SATTN_QK_SMOOTH_Q.
bool valid_format(int f) {
  const int base = f & ~SATTN_QK_SMOOTH_Q;
  return base == SATTN_QK_INT8 || base == SATTN_QK_FP8;
}
bool is_fp8(int f) { return (f & ~SATTN_QK_SMOOTH_Q) == SATTN_QK_FP8; }
bool is_qsmooth(int f) { return (f & SATTN_QK_SMOOTH_Q) != 0; }

// Q smoothing in the E4M3 Q/K format adds a Delta-S table of
// B*H*nbq*nbk*128 floats; past 2^40 bytes (far beyond device memory) the
// sizes are refused.
sattn_status check_qsmooth(int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int f) {
  if (!is_qsmooth(f) || !is_fp8(f)) return SATTN_OK;
  const double bytes = (double)B * (double)H * (double)sattn::nblocks(Nq) * (double)sattn::nblocks(Nkv) * 512.0;
  return bytes > 1099511627776.0 ? SATTN_ERR_UNSUPPORTED : SATTN_OK;
}

// Split-KV: how many key-tile ranges, and tiles per range, for a request of
// num_splits (0: automatic).  The automatic choice splits only a launch whose
// workgroups (B*H*ceil(Nq/256), one per CU at a time) would not fill the 256
// CUs of an MI355X once, into as many ranges as fill them, each of at least
// kMinTilesPerSplit key tiles.  Every range holds at least one tile.
constexpr int64_t kCUs = 256;
constexpr int64_t kMinTilesPerSplit = 8;

struct Split {
  int splits, tps;
};

Split resolve_splits(int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int num_splits) {
  const int64_t nbk = sattn::nblocks(Nkv);
  int64_t want = num_splits;
  if (want == 0) {
    const int64_t g1 = B * H * ((Nq + 255) / 256);
    want = 1;
    if (g1 < kCUs) {
      want = kCUs / g1;
      if (want > nbk / kMinTilesPerSplit) want = nbk / kMinTilesPerSplit;
      if (want < 1) want = 1;
    }
  }
  if (want > nbk) want = nbk;
  const int64_t tps = (nbk + want - 1) / want;
  return {(int)((nbk + tps - 1) / tps), (int)tps};
}

sattn_status fwd_common(const void* packed, size_t packed_bytes, int qk_format, int64_t B, int64_t H,
                        int64_t Nq, int64_t Nkv, int64_t D, float softmax_scale, void* out,
                        const int64_t* out_strides, float* lse, int num_splits, void* workspace,
                        size_t workspace_bytes, void* stream, bool cross,
                        const void* lut = nullptr, size_t lut_bytes = 0) {
  sattn_status s = check_dims(B, H, Nq, Nkv, D);
  if (s != SATTN_OK) return s;
  if (!valid_format(qk_format)) return SATTN_ERR_INVALID_ARGUMENT;
  if ((s = check_qsmooth(B, H, Nq, Nkv, qk_format)) != SATTN_OK) return s;
  if (lut != nullptr && is_qsmooth(qk_format)) return SATTN_ERR_UNSUPPORTED;
  if (num_splits < 0 || num_splits > SATTN_MAX_SPLITS) return SATTN_ERR_INVALID_ARGUMENT;
  if (packed == nullptr || out == nullptr) return SATTN_ERR_INVALID_ARGUMENT;
  if (!aligned16(packed) || !aligned16(out)) return SATTN_ERR_INVALID_ARGUMENT;
  if (lse != nullptr && ((uintptr_t)lse & 3u) != 0) return SATTN_ERR_INVALID_ARGUMENT;
  const Split sp = lut != nullptr ? Split{1, (int)sattn::nblocks(Nkv)}
                                  : resolve_splits(B, H, Nq, Nkv, num_splits);
  if (lut != nullptr) {
    if (!aligned16(lut)) return SATTN_ERR_INVALID_ARGUMENT;
    if (lut_bytes < (size_t)sattn::block_lut_bytes(B, H, Nq, sattn::nblocks(Nkv)))
      return SATTN_ERR_BUFFER_TOO_SMALL;
  }
  if (sp.splits > 1) {
    if (workspace == nullptr || !aligned16(workspace)) return SATTN_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < (size_t)sattn::split_workspace_bytes(sp.splits, B * H, Nq))
      return SATTN_ERR_BUFFER_TOO_SMALL;
  }
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.0f)) return SATTN_ERR_INVALID_ARGUMENT;
  sattn::AttnArgs a;
  s = get_strides(out_strides, Nq, H, a.o_str);
  if (s != SATTN_OK) return s;
  a.L = sattn::make_layout(B, H, Nq, Nkv, is_qsmooth(qk_format), is_fp8(qk_format));
  if (packed_bytes < a.L.packed_bytes) return SATTN_ERR_BUFFER_TOO_SMALL;
  s = check_device();
  if (s != SATTN_OK) return s;
  a.packed = static_cast<const uint8_t*>(packed);
  a.softmax_scale = softmax_scale;
  a.out = static_cast<uint16_t*>(out);
  a.fp8qk = is_fp8(qk_format);
  a.lse = lse;
  a.splits = sp.splits;
  a.tps = sp.tps;
  a.workspace = static_cast<uint8_t*>(workspace);
  a.lut_counts = nullptr;
  a.lut_entries = nullptr;
  if (lut != nullptr) {
    const uint8_t* l = static_cast<const uint8_t*>(lut);
    a.lut_counts = reinterpret_cast<const int32_t*>(l);
    a.lut_entries = reinterpret_cast<const uint32_t*>(
        l + sattn::lut_counts_bytes(B * H * ((Nq + 255) / 256)));
  }
  return launch_status(sattn::launch_attention(a, cross, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int sattn_abi_version(void) { return SATTN_ABI_VERSION; }

const char* sattn_status_string(int status) {
  switch (status) {
    case SATTN_OK: return "ok";
    case SATTN_ERR_INVALID_ARGUMENT: return "invalid argument";
    case SATTN_ERR_UNSUPPORTED: return "unsupported";
    case SATTN_ERR_BUFFER_TOO_SMALL: return "buffer too small";
    case SATTN_ERR_DEVICE: return "no gfx950 device";
    case SATTN_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

sattn_status sattn_packed_bytes_ex(int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t D, int qk_format,
                                   size_t* packed_bytes, size_t* workspace_bytes) {
  sattn_status s = check_dims(B, H, Nq, Nkv, D);
  if (s != SATTN_OK) return s;
  if (!valid_format(qk_format)) return SATTN_ERR_INVALID_ARGUMENT;
  if ((s = check_qsmooth(B, H, Nq, Nkv, qk_format)) != SATTN_OK) return s;
  const Layout L = sattn::make_layout(B, H, Nq, Nkv, is_qsmooth(qk_format), is_fp8(qk_format));
  if (packed_bytes) *packed_bytes = L.packed_bytes;
  if (workspace_bytes) *workspace_bytes = L.workspace_bytes;
  return SATTN_OK;
}

sattn_status sattn_packed_bytes(int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t D,
                                size_t* packed_bytes, size_t* workspace_bytes) {
  return sattn_packed_bytes_ex(B, H, Nq, Nkv, D, SATTN_QK_INT8, packed_bytes, workspace_bytes);
}

}  // extern "C"

namespace {

// Shared by the quantize entry points.  workspace == nullptr with
// use_static: the library's static workspace (sattn_quantize_qkv_noalloc).
sattn_status quantize_common(const void* q, const void* k, const void* v, int64_t B, int64_t H, int64_t Nq,
                             int64_t Nkv, int64_t D, const int64_t* q_strides, const int64_t* k_strides,
                             const int64_t* v_strides, int qk_format, void* packed, size_t packed_bytes,
                             void* workspace, size_t workspace_bytes, bool use_static, void* stream) {
  sattn_status s = check_dims(B, H, Nq, Nkv, D);
  if (s != SATTN_OK) return s;
  if (!valid_format(qk_format)) return SATTN_ERR_INVALID_ARGUMENT;
  if ((s = check_qsmooth(B, H, Nq, Nkv, qk_format)) != SATTN_OK) return s;
  if (!q || !k || !v || !packed || (!use_static && !workspace)) return SATTN_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(packed) ||
      (!use_static && !aligned16(workspace)))
    return SATTN_ERR_INVALID_ARGUMENT;
  sattn::QuantArgs a;
  if ((s = get_strides(q_strides, Nq, H, a.q_str)) != SATTN_OK) return s;
  if ((s = get_strides(k_strides, Nkv, H, a.k_str)) != SATTN_OK) return s;
  if ((s = get_strides(v_strides, Nkv, H, a.v_str)) != SATTN_OK) return s;
  a.L = sattn::make_layout(B, H, Nq, Nkv, is_qsmooth(qk_format), is_fp8(qk_format));
  if (packed_bytes < a.L.packed_bytes) return SATTN_ERR_BUFFER_TOO_SMALL;
  if (use_static ? a.L.workspace_bytes > SATTN_NOALLOC_WORKSPACE_BYTES : workspace_bytes < a.L.workspace_bytes)
    return use_static ? SATTN_ERR_UNSUPPORTED : SATTN_ERR_BUFFER_TOO_SMALL;
  s = check_device();
  if (s != SATTN_OK) return s;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  if (use_static && sattn::noalloc_workspace(&ws) != hipSuccess) return SATTN_ERR_DEVICE;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.packed = static_cast<uint8_t*>(packed);
  a.workspace = ws;
  a.fp8qk = is_fp8(qk_format);
  return launch_status(sattn::launch_quantize(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

sattn_status sattn_quantize_qkv_ex(const void* q, const void* k, const void* v,
                                   int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t D,
                                   const int64_t* q_strides, const int64_t* k_strides,
                                   const int64_t* v_strides, int qk_format,
                                   void* packed, size_t packed_bytes,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  return quantize_common(q, k, v, B, H, Nq, Nkv, D, q_strides, k_strides, v_strides, qk_format, packed,
                         packed_bytes, workspace, workspace_bytes, false, stream);
}

sattn_status sattn_quantize_qkv_noalloc(const void* q, const void* k, const void* v,
                                        int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t D,
                                        const int64_t* q_strides, const int64_t* k_strides,
                                        const int64_t* v_strides, int qk_format,
                                        void* packed, size_t packed_bytes, void* stream) {
  return quantize_common(q, k, v, B, H, Nq, Nkv, D, q_strides, k_strides, v_strides, qk_format, packed,
                         packed_bytes, nullptr, 0, true, stream);
}

sattn_status sattn_quantize_qkv(const void* q, const void* k, const void* v,
                                int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t D,
                                const int64_t* q_strides, const int64_t* k_strides,
                                const int64_t* v_strides,
                                void* packed, size_t packed_bytes,
                                void* workspace, size_t workspace_bytes, void* stream) {
  return sattn_quantize_qkv_ex(q, k, v, B, H, Nq, Nkv, D, q_strides, k_strides, v_strides,
                               SATTN_QK_INT8, packed, packed_bytes, workspace, workspace_bytes,
                               stream);
}

sattn_status sattn_fwd_workspace_bytes(int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t D,
                                       int num_splits, size_t* workspace_bytes, int* splits_used) {
  sattn_status s = check_dims(B, H, Nq, Nkv, D);
  if (s != SATTN_OK) return s;
  if (num_splits < 0 || num_splits > SATTN_MAX_SPLITS) return SATTN_ERR_INVALID_ARGUMENT;
  const Split sp = resolve_splits(B, H, Nq, Nkv, num_splits);
  if (workspace_bytes) *workspace_bytes = (size_t)sattn::split_workspace_bytes(sp.splits, B * H, Nq);
  if (splits_used) *splits_used = sp.splits;
  return SATTN_OK;
}

sattn_status sattn_fwd_ex(const void* packed, size_t packed_bytes, int qk_format, int64_t B,
                          int64_t H, int64_t N, int64_t D, float softmax_scale, void* out,
                          const int64_t* out_strides, float* lse, int num_splits, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return fwd_common(packed, packed_bytes, qk_format, B, H, N, N, D, softmax_scale, out, out_strides,
                    lse, num_splits, workspace, workspace_bytes, stream, false);
}

sattn_status sattn_fwd_cross_ex(const void* packed, size_t packed_bytes, int qk_format, int64_t B,
                                int64_t H, int64_t Nq, int64_t Nkv, int64_t D, float softmax_scale,
                                void* out, const int64_t* out_strides, float* lse, int num_splits,
                                void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_common(packed, packed_bytes, qk_format, B, H, Nq, Nkv, D, softmax_scale, out,
                    out_strides, lse, num_splits, workspace, workspace_bytes, stream, true);
}

sattn_status sattn_block_lut_bytes(int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t D,
                                   size_t* lut_bytes) {
  sattn_status s = check_dims(B, H, Nq, Nkv, D);
  if (s != SATTN_OK) return s;
  if (lut_bytes) *lut_bytes = (size_t)sattn::block_lut_bytes(B, H, Nq, sattn::nblocks(Nkv));
  return SATTN_OK;
}

sattn_status sattn_block_lut(const uint8_t* block_mask, int64_t B, int64_t H, int64_t Nq, int64_t Nkv,
                             int64_t D, void* lut, size_t lut_bytes, void* stream) {
  sattn_status s = check_dims(B, H, Nq, Nkv, D);
  if (s != SATTN_OK) return s;
  if (block_mask == nullptr || lut == nullptr || !aligned16(lut)) return SATTN_ERR_INVALID_ARGUMENT;
  if (lut_bytes < (size_t)sattn::block_lut_bytes(B, H, Nq, sattn::nblocks(Nkv)))
    return SATTN_ERR_BUFFER_TOO_SMALL;
  s = check_device();
  if (s != SATTN_OK) return s;
  const Layout L = sattn::make_layout(B, H, Nq, Nkv);
  return launch_status(sattn::launch_block_lut(block_mask, L, static_cast<uint8_t*>(lut),
                                               static_cast<hipStream_t>(stream)));
}

sattn_status sattn_fwd_sparse(const void* packed, size_t packed_bytes, int qk_format, int64_t B,
                              int64_t H, int64_t Nq, int64_t Nkv, int64_t D, float softmax_scale,
                              const void* lut, size_t lut_bytes, void* out,
                              const int64_t* out_strides, float* lse, void* stream) {
  if (lut == nullptr) return SATTN_ERR_INVALID_ARGUMENT;
  return fwd_common(packed, packed_bytes, qk_format, B, H, Nq, Nkv, D, softmax_scale, out, out_strides,
                    lse, 1, nullptr, 0, stream, true, lut, lut_bytes);
}

sattn_status sattn_fwd(const void* packed, size_t packed_bytes, int64_t B, int64_t H, int64_t N,
                       int64_t D, float softmax_scale, void* out, const int64_t* out_strides,
                       void* stream) {
  return sattn_fwd_ex(packed, packed_bytes, SATTN_QK_INT8, B, H, N, D, softmax_scale, out,
                      out_strides, nullptr, 1, nullptr, 0, stream);
}

sattn_status sattn_fwd_cross(const void* packed, size_t packed_bytes, int64_t B, int64_t H,
                             int64_t Nq, int64_t Nkv, int64_t D, float softmax_scale, void* out,
                             const int64_t* out_strides, void* stream) {
  return sattn_fwd_cross_ex(packed, packed_bytes, SATTN_QK_INT8, B, H, Nq, Nkv, D, softmax_scale,
                            out, out_strides, nullptr, 1, nullptr, 0, stream);
}

sattn_status sattn_unpack_host(const void* packed_host, size_t packed_bytes, int64_t B, int64_t H,
                               int64_t Nq, int64_t Nkv, int64_t D, int8_t* q8, int8_t* k8,
                               uint8_t* v8, float* q_scale, float* k_scale, float* v_scale,
                               float* k_mean) {
  sattn_status s = check_dims(B, H, Nq, Nkv, D);
  if (s != SATTN_OK) return s;
  if (packed_host == nullptr) return SATTN_ERR_INVALID_ARGUMENT;
  const Layout L = sattn::make_layout(B, H, Nq, Nkv);
  if (packed_bytes < L.packed_bytes) return SATTN_ERR_BUFFER_TOO_SMALL;
  const uint8_t* P = static_cast<const uint8_t*>(packed_host);
  const int64_t BH = B * H;
  for (int64_t bh = 0; bh < BH; ++bh) {
    if (q8)
      for (int64_t n = 0; n < Nq; ++n) {
        const uint8_t* tile = P + L.off_q8 + (bh * L.nbq + n / 128) * sattn::kTileBytes;
        for (int c = 0; c < 128; ++c)
          q8[(bh * Nq + n) * 128 + c] = (int8_t)tile[sattn::q_pos((int)(n % 128), c)];
      }
    if (k8)
      for (int64_t n = 0; n < Nkv; ++n) {
        const uint8_t* tile = P + L.off_k8 + (bh * L.nbk + n / 128) * sattn::kTileBytes;
        for (int c = 0; c < 128; ++c)
          k8[(bh * Nkv + n) * 128 + c] = (int8_t)tile[sattn::k_pos((int)(n % 128), c)];
      }
    if (v8)
      for (int64_t n = 0; n < Nkv; ++n) {
        const uint8_t* tile = P + L.off_v8 + (bh * L.nbk + n / 128) * sattn::kTileBytes;
        for (int d = 0; d < 128; ++d) v8[(bh * Nkv + n) * 128 + d] = tile[sattn::v_pos((int)(n % 128), d)];
      }
  }
  if (q_scale) memcpy(q_scale, P + L.off_qs, (size_t)BH * L.nbq * 4);
  if (k_scale) memcpy(k_scale, P + L.off_ks, (size_t)BH * L.nbk * 4);
  if (v_scale) memcpy(v_scale, P + L.off_vs, (size_t)BH * 128 * 4);
  if (k_mean) memcpy(k_mean, P + L.off_km, (size_t)BH * 128 * 4);
  return SATTN_OK;
}

sattn_status sattn_unpack_q_mean_host(const void* packed_host, size_t packed_bytes, int64_t B, int64_t H,
                                      int64_t Nq, int64_t Nkv, int64_t D, float* q_mean) {
  sattn_status s = check_dims(B, H, Nq, Nkv, D);
  if (s != SATTN_OK) return s;
  if ((s = check_qsmooth(B, H, Nq, Nkv, SATTN_QK_SMOOTH_Q)) != SATTN_OK) return s;
  if (packed_host == nullptr || q_mean == nullptr) return SATTN_ERR_INVALID_ARGUMENT;
  const Layout L = sattn::make_layout(B, H, Nq, Nkv, true);
  const size_t bytes = (size_t)(B * H * L.nbq) * 128 * 4;
  if (packed_bytes < L.off_qm + bytes) return SATTN_ERR_BUFFER_TOO_SMALL;
  memcpy(q_mean, static_cast<const uint8_t*>(packed_host) + L.off_qm, bytes);
  return SATTN_OK;
}

sattn_status sattn_e4m3_encode(const float* x, uint8_t* out, int64_t n, void* stream) {
  if (x == nullptr || out == nullptr || n <= 0 || n > kMaxElems) return SATTN_ERR_INVALID_ARGUMENT;
  sattn_status s = check_device();
  if (s != SATTN_OK) return s;
  return launch_status(sattn::launch_e4m3_encode(x, out, n, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
