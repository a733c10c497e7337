/*
 * sattn.h -- C ABI of libsattn: INT8-QK / FP8-PV ("SageAttention-style")
 * dense attention forward for MI355X (gfx950).
 *
 * The operation.  Multi-head attention O = softmax(scale * Q K^T) V with
 * head dimension 128, non-causal, no mask, no dropout, BF16 Q/K/V in and BF16
 * out, computed with an INT8 Q.K^T contraction, an FP8 P.V contraction and
 * FP32 accumulation.  This is the operand contract of the gfx1201 backend
 * page ("[ROCm] Add aiter_sage_attn attention backend for gfx1201 (RDNA4)",
 * section "Changes") and the INT8/FP8/BF16 row of the MI355X throughput table
 * of "new MHA v4 entrypoint; hosts a spectrum of quantized & sparse attention
 * kernels" (Test Result).  As on that page (Technical Details), Q/K/V
 * preprocessing is a separate call that writes an opaque packed buffer whose
 * size is queried first; the attention calls consume it.
 *
 * Quantization (the method's definition; the pages name the formats only):
 *   - Q: per (batch, head, 128-token block) scale qs = amax|q| / 127 (FP32),
 *     code = clamp(round-half-even(q / qs), -127, 127); qs == 0 -> codes 0.
 *   - K: mean-smoothed.  mean[d] = (sum over 128-token blocks, in block
 *     order, of the FP32 sum of the block's tokens in token order) / Nkv;
 *     k' = fl32(k - mean); then per block as for Q.
 *   - V: per (batch, head, channel) scale vs = amax|v| / 448, code = OCP
 *     E4M3 round-to-nearest-even of clamp(v / vs, -448, 448); the sign of
 *     zero is kept.  All divisions are correctly rounded FP32 divisions.
 *   - Attention: S = (q8 . k8) * qs * ks * scale, online softmax in base 2,
 *     P quantized as E4M3(448 p) against the running row maximum, O
 *     accumulated in FP32 from FP8 P and FP8 V, row sum l from FP32 p,
 *     O = acc * vs / (448 l) rounded to BF16.
 *
 * Conventions shared by every entry point.
 *   - All device pointers are caller-owned (hipMalloc or a framework
 *     allocator).  The library never allocates, frees or synchronizes; the
 *     only state it keeps is a per-device architecture check.  Calls are
 *     reentrant and stream-ordered on `stream` (a hipStream_t; NULL is the
 *     default stream); they may be captured into a HIP graph.
 *   - BF16 tensors are addressed as [B, N, H, 128] with element strides
 *     (batch, sequence, head) given by a 3-entry array; the last dimension is
 *     contiguous.  NULL strides mean contiguous BSHD (N*H*128, H*128, 128).
 *     Base pointers must be 16-byte aligned and strides multiples of 8.
 *   - Errors: every argument is validated before any HIP call; on error
 *     nothing is read or written, nothing is launched and the status says
 *     why.  There is no fallback path.  Unsupported features (D != 128, a
 *     non-gfx950 device) are errors, never a different computation.
 */
#ifndef SATTN_H
#define SATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SATTN_ABI_VERSION 2
#define SATTN_HEAD_DIM 128
#define SATTN_BLOCK 128
/* longest supported sequence (keeps the K mean divisor exact in FP32) */
#define SATTN_MAX_SEQ (1 << 24)
/* largest B * H * ceil(max(Nq, Nkv) / 128): keeps every launch's grid within
   32-bit work-item counts (2^22 blocks are 2^36 elements per tensor, more
   than one GPU's memory holds) */
#define SATTN_MAX_BLOCKS (1 << 22)
/* largest num_splits of the split-KV forward calls */
#define SATTN_MAX_SPLITS 256
/* Size of the static workspace of sattn_quantize_qkv_noalloc (16 MiB per
   device; enough for B*H*ceil(Nkv/128) <= 16384). */
#define SATTN_NOALLOC_WORKSPACE_BYTES ((size_t)16 << 20)

typedef enum {
  SATTN_OK = 0,
  SATTN_ERR_INVALID_ARGUMENT = 1, /* null or misaligned pointer, size <= 0, size overflow,
                                     bad stride, softmax_scale not finite and > 0 */
  SATTN_ERR_UNSUPPORTED = 2,      /* D != 128; sattn_fwd with Nq != Nkv; N > SATTN_MAX_SEQ;
                                     more than SATTN_MAX_BLOCKS blocks */
  SATTN_ERR_BUFFER_TOO_SMALL = 3, /* packed or workspace bytes below the queried size */
  SATTN_ERR_DEVICE = 4,           /* no HIP device, or the current device is not gfx950 */
  SATTN_ERR_LAUNCH = 5            /* a kernel launch reported an error */
} sattn_status;

/*
 * Q/K code formats.  SATTN_QK_INT8: INT8 codes with block scale amax/127
 * (the INT8/FP8/BF16 path of the gfx1201 backend page, "Changes").
 * SATTN_QK_FP8: OCP E4M3 codes with block scale amax/448 and an FP8 Q.K^T
 * MFMA (the FP8/FP8/BF16 row of the MHA v4 page's MI355X throughput table).
 * V and P are E4M3 in both.  The entry points without a format argument use
 * SATTN_QK_INT8.
 */
typedef enum { SATTN_QK_INT8 = 0, SATTN_QK_FP8 = 1 } sattn_qk_format;

/*
 * Option OR-ed into a qk_format: Q smoothing with the Delta-S correction
 * (the MHA v4 page's import listing names a Q-smoothing kernel and a
 * Delta-S kernel).  Per (b, h, 128-token Q block) the FP32 mean of the
 * block's tokens (token order, one division by their count) is subtracted
 * before the block is coded, and every score gets back Delta-S = ks(j) *
 * (q_mean . kcode_j) * softmax_scale.  The packed buffer then also holds the
 * means (size from sattn_packed_bytes_ex) and:
 *   - with SATTN_QK_INT8, per Q block four int8 digit rows of the mean in
 *     the block's score unit and 8 parameters (512 + 32 bytes); the forward
 *     forms Delta-S on the INT8 MFMA from them, rounded to the score unit
 *     (qs; a coarser unit qs * 2^k, with the block's Q codes rounded to it,
 *     only where the mean exceeds 2^15 code units), as the initial value of
 *     the score accumulators;
 *   - with SATTN_QK_FP8, a Delta-S table of B*H*ceil(Nq/128)*ceil(Nkv/128)*
 *     128 floats, added to each score by the forward.
 * Not with sattn_fwd_sparse.
 */
#define SATTN_QK_SMOOTH_Q 0x10

/* ABI version of the loaded library (SATTN_ABI_VERSION). */
int sattn_abi_version(void);

/* Static, human-readable name of a status code (a sattn_status value);
   any other value gives "unknown status".  Taken as int so that an
   out-of-range value is well defined on both sides of the call. */
const char* sattn_status_string(int status);

/*
 * Sizes of the two caller-owned device buffers for a problem:
 *   packed_bytes    -- output of sattn_quantize_qkv, input of the forward
 *                      calls: Q8, K8 and V8 tiles plus all scales and the K
 *                      mean, 256-byte aligned sections.
 *   workspace_bytes -- scratch for the per-block K sums and V maxima
 *                      (contents undefined between calls).
 * Either output pointer may be NULL.  Pure host function; no device needed.
 */
sattn_status sattn_packed_bytes(int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t D,
                                size_t* packed_bytes, size_t* workspace_bytes);
/* The same for a qk_format (a format, optionally | SATTN_QK_SMOOTH_Q). */
sattn_status sattn_packed_bytes_ex(int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t D, int qk_format,
                                   size_t* packed_bytes, size_t* workspace_bytes);

/*
 * Preprocessing: quantize BF16 q [B,Nq,H,128], k and v [B,Nkv,H,128] into
 * `packed` (the INT8/E4M3 codes in the tile order the attention kernels load
 * into LDS, the Q/K block scales, the V channel scales and the K mean).
 * Launches three kernels on `stream`: per-block K sums and V maxima into
 * `workspace`; the K mean and V scales; the codes.  The result does not
 * depend on softmax_scale, so one packed buffer serves any scale.
 */
sattn_status sattn_quantize_qkv(const void* q, const void* k, const void* v,
                                int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t D,
                                const int64_t* q_strides, const int64_t* k_strides,
                                const int64_t* v_strides,
                                void* packed, size_t packed_bytes,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Self-attention forward from a packed buffer made with Nq == Nkv == N.
 * softmax_scale: positive, finite (callers pass 1/sqrt(128) for the usual
 * scaling).  out: BF16 [B,N,H,128] with `out_strides` (NULL = contiguous).
 * Nq != Nkv is SATTN_ERR_UNSUPPORTED (use sattn_fwd_cross).
 */
sattn_status sattn_fwd(const void* packed, size_t packed_bytes,
                       int64_t B, int64_t H, int64_t N, int64_t D, float softmax_scale,
                       void* out, const int64_t* out_strides, void* stream);

/*
 * Cross-attention forward: any Nq, Nkv >= 1 (tuned for short key sequences
 * such as 512 text tokens); same conventions as sattn_fwd.  The packed buffer
 * must have been made with the same (B, H, Nq, Nkv).
 */
sattn_status sattn_fwd_cross(const void* packed, size_t packed_bytes,
                             int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t D,
                             float softmax_scale, void* out, const int64_t* out_strides,
                             void* stream);

/*
 * The same three calls with the Q/K code format as an argument, and for the
 * forward calls an optional LSE output and split-KV.
 *
 * qk_format: a sattn_qk_format, optionally | SATTN_QK_SMOOTH_Q; another value
 *   is SATTN_ERR_INVALID_ARGUMENT.
 *   The packed layout and its size are the same for both formats; a packed
 *   buffer must be read with the format it was written with (the library
 *   cannot tell them apart).
 *
 * lse: NULL, or device FP32 [B][H][Nq] contiguous (4-byte aligned): per query
 *   row the natural-log log-sum-exp of its logits before K smoothing,
 *   m + ln(l) over the smoothed scores plus softmax_scale * qs *
 *   sum_d qcode_d * kmean_d (the shift the smoothing removed).  It estimates
 *   ln sum_j exp(softmax_scale * q . k_j), so outputs over disjoint key sets
 *   merge as O = sum_i exp(lse_i - lse) O_i with lse = ln sum_i exp(lse_i)
 *   (the float32 LSE and split-KV of the FA4 autotuning page, "Validation").
 *
 * num_splits: 1 = one workgroup sweeps all keys of its queries (the calls
 *   without these arguments); k in [2, SATTN_MAX_SPLITS] = the key tiles are
 *   cut into at most k ranges swept by separate workgroups, whose FP32
 *   partial outputs and LSE are merged by a second kernel with the rule
 *   above (for few queries and many keys, where one range per query tile
 *   leaves most CUs idle); 0 = the library's choice (splits only launches
 *   that would not fill the device once).  Other values are
 *   SATTN_ERR_INVALID_ARGUMENT.
 * workspace: device memory of at least the size sattn_fwd_workspace_bytes
 *   returns for the same (B, H, Nq, Nkv, D, num_splits), 16-byte aligned,
 *   caller-owned, not read before it is written; may be NULL (size 0) when
 *   that size is 0.  Too small is SATTN_ERR_BUFFER_TOO_SMALL.
 */
sattn_status sattn_quantize_qkv_ex(const void* q, const void* k, const void* v,
                                   int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t D,
                                   const int64_t* q_strides, const int64_t* k_strides,
                                   const int64_t* v_strides, int qk_format,
                                   void* packed, size_t packed_bytes,
                                   void* workspace, size_t workspace_bytes, void* stream);
/*
 * sattn_quantize_qkv_ex without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, serving
 * loops and harnesses that forbid allocation): the per-block K sums and V
 * maxima go to a static device array of SATTN_NOALLOC_WORKSPACE_BYTES, one
 * per GPU, held by the library until the process ends.  The call allocates
 * nothing; the caller still passes inputs and `packed`.  Results are those
 * of sattn_quantize_qkv_ex bit for bit.
 * Errors as sattn_quantize_qkv_ex, plus SATTN_ERR_UNSUPPORTED when the
 * problem's workspace (sattn_packed_bytes) exceeds the static array, and
 * SATTN_ERR_DEVICE when its device address cannot be obtained.  Every call
 * on one GPU uses the same array: calls that overlap on a GPU (other
 * streams, other host threads) race and must be serialised by the caller.
 */
sattn_status sattn_quantize_qkv_noalloc(const void* q, const void* k, const void* v,
                                        int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t D,
                                        const int64_t* q_strides, const int64_t* k_strides,
                                        const int64_t* v_strides, int qk_format,
                                        void* packed, size_t packed_bytes, void* stream);
sattn_status sattn_fwd_ex(const void* packed, size_t packed_bytes, int qk_format,
                          int64_t B, int64_t H, int64_t N, int64_t D, float softmax_scale,
                          void* out, const int64_t* out_strides, float* lse, int num_splits,
                          void* workspace, size_t workspace_bytes, void* stream);
sattn_status sattn_fwd_cross_ex(const void* packed, size_t packed_bytes, int qk_format,
                                int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t D,
                                float softmax_scale, void* out, const int64_t* out_strides,
                                float* lse, int num_splits, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * Host-only size query for the split-KV workspace: bytes of workspace and
 * the number of key ranges the forward calls will use for this problem and
 * num_splits (either output pointer may be NULL).  Size 0 means no split.
 */
sattn_status sattn_fwd_workspace_bytes(int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t D,
                                       int num_splits, size_t* workspace_bytes, int* splits_used);

/*
 * Block-sparse attention (the MHA v4 page's block-mask-to-ragged-LUT
 * conversion and block-sparse reference; the sparse pipelines the AITER bump
 * page measures).  Query i attends key j iff
 * block_mask[b][h][i / 128][j / 128] != 0: 128-token blocks on both sides,
 * the quantization blocks.  The quantizer does not see the mask; softmax, P
 * rounding and the LSE run over each row's allowed keys; a row with no
 * allowed key gets output 0 and lse -inf.
 *
 * sattn_block_lut_bytes: host-only size of the table for a problem.
 * sattn_block_lut: block_mask = device uint8 [B][H][ceil(Nq/128)][ceil(Nkv/128)]
 *   -> `lut` (device, caller-owned, 16-byte aligned, at least that size):
 *   per tile of 256 queries (query blocks 2m and 2m+1) the ascending list of
 *   the key blocks either attends, each entry marking which of the two does.
 *   Launches one kernel on `stream`.  The table layout is the library's own;
 *   pass it only to sattn_fwd_sparse with the same (B, H, Nq, Nkv).
 * sattn_fwd_sparse: attention over the listed blocks (any Nq, Nkv), with
 *   the conventions of sattn_fwd_cross_ex (qk_format, lse; no split-KV).
 *   Work scales with the listed blocks.  Entries and counts are clamped to
 *   the problem, so a damaged table gives wrong output, never an access
 *   outside the buffers.
 */
sattn_status sattn_block_lut_bytes(int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t D,
                                   size_t* lut_bytes);
sattn_status sattn_block_lut(const uint8_t* block_mask, int64_t B, int64_t H, int64_t Nq, int64_t Nkv,
                             int64_t D, void* lut, size_t lut_bytes, void* stream);
sattn_status sattn_fwd_sparse(const void* packed, size_t packed_bytes, int qk_format,
                              int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t D,
                              float softmax_scale, const void* lut, size_t lut_bytes,
                              void* out, const int64_t* out_strides, float* lse, void* stream);

/*
 * Host-only: the Q block means [B][H][ceil(Nq/128)][128] FP32 of a host copy
 * of a packed buffer quantized with SATTN_QK_SMOOTH_Q.
 */
sattn_status sattn_unpack_q_mean_host(const void* packed_host, size_t packed_bytes, int64_t B, int64_t H,
                                      int64_t Nq, int64_t Nkv, int64_t D, float* q_mean);

/*
 * Host-only inspection of a packed buffer (a host copy of it): writes the
 * canonical layouts
 *   q8 [B,H,Nq,128] and k8 [B,H,Nkv,128] (INT8 codes, or E4M3 bits for
 *   SATTN_QK_FP8), v8 [B,H,Nkv,128] E4M3 bits,
 *   q_scale [B,H,ceil(Nq/128)], k_scale [B,H,ceil(Nkv/128)],
 *   v_scale [B,H,128], k_mean [B,H,128] (FP32).
 * Any output pointer may be NULL to skip it.  No device needed.
 */
sattn_status sattn_unpack_host(const void* packed_host, size_t packed_bytes,
                               int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t D,
                               int8_t* q8, int8_t* k8, uint8_t* v8,
                               float* q_scale, float* k_scale, float* v_scale, float* k_mean);

/*
 * The device FP32 -> OCP E4M3 conversion used by the V quantizer, applied
 * elementwise: out[i] = E4M3_RNE(clamp(x[i], -448, 448)), sign of zero kept
 * (x must not be NaN).  x: n FP32 values, out: n bytes, both device pointers;
 * n >= 1.  Exposed so that the conversion can be checked exhaustively.
 */
sattn_status sattn_e4m3_encode(const float* x, uint8_t* out, int64_t n, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SATTN_H */
