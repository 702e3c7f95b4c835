/*
 * skiparse.h -- C ABI of libskiparse, Skiparse-2D sparse attention forward on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (OSP-Next summary page, 核心方法 "core method" and
 * 方法步骤详情 "method steps"; OSP-Next abstract):
 *   video tokens (B, T, H, W, heads, d) are regrouped by a fixed rule into k*k
 *   independent subsequences; dense softmax attention runs inside each
 *   subsequence; every output row is written back at its token's original
 *   position.
 *     token-wise  (pixel unshuffle): token (h, w) joins subsequence
 *                 s = (h mod k) * k + (w mod k);
 *     group-wise  (patch unshuffle of k x k blocks, block index mod k):
 *                 s = ((h / k) mod k) * k + ((w / k) mod k).
 *   When H or W is not a multiple of k*k the grid is padded at the high end
 *   to the next multiple and the padded tokens are masked (any-resolution
 *   rule), so that a position follows the same pattern at every resolution.
 *   k = 1 is plain full attention (the hybrid model's full-attention layers).
 *
 * Conventions for every entry point:
 *   - Device pointers are HIP device memory owned by the caller; the library
 *     never allocates, frees or synchronizes.  All device work is enqueued on
 *     the given stream and runs asynchronously.
 *   - Tensors are contiguous (B, T, H, W, heads, d), row-major, 16-byte
 *     aligned base pointers.
 *   - Return value: SKIPARSE_OK (0) or a negative skiparse_status.  Arguments
 *     are validated before anything is launched; on error nothing is
 *     enqueued and skiparse_last_error() describes the problem.
 *   - Thread safety: the library keeps no state apart from a thread-local
 *     error string.
 */
#ifndef SKIPARSE_H
#define SKIPARSE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SKIPARSE_ABI_VERSION 1
#define SKIPARSE_MAX_K 8

typedef enum {
  SKIPARSE_OK = 0,
  SKIPARSE_EINVAL = -1,        /* bad argument: null or misaligned pointer, bad size */
  SKIPARSE_EUNSUPPORTED = -2,  /* valid but not built: d not in {64, 128}, k > 8, ... */
  SKIPARSE_EHIP = -3,          /* the HIP runtime reported an error at launch */
  SKIPARSE_EWORKSPACE = -4     /* workspace missing or too small */
} skiparse_status;

typedef enum {
  SKIPARSE_MODE_TOKEN = 0,     /* token-wise pattern */
  SKIPARSE_MODE_GROUP = 1,     /* group-wise pattern (ignored when k == 1) */
  /* Skiparse-1D, the variant the 2D pattern is compared with (OSP-Next
   * summary, novelty): the same two rules on each frame's flattened spatial
   * index l = h*W + w, stride k*k (density 1/k^2 as in 2D), l padded at its
   * end to a multiple of k^4; every subsequence spans all T frames.  The plan
   * then describes the grid (T, 1, H*W): Hp = 1, Wp = padded length,
   * sub_h = 1, sub_w = Wp / k^2, real_h[0] = 1, real_w[q] for q < k^2, and
   * subsequence s = q.  k <= 2 (k^2 extents must fit real_w). */
  SKIPARSE_MODE_TOKEN_1D = 2,
  SKIPARSE_MODE_GROUP_1D = 3
} skiparse_mode;

typedef enum {
  SKIPARSE_F32 = 0,            /* fp32 in, fp32 out */
  SKIPARSE_BF16 = 1,           /* bf16 in, bf16 out, fp32 accumulation */
  SKIPARSE_FP8_E4M3 = 2        /* OCP e4m3 in (per-tensor scaled), bf16 out */
} skiparse_dtype;

/*
 * Geometry of one attention call, filled by skiparse_plan_init.  Plain data:
 * the caller owns it and may copy it.
 *   Hp, Wp          H, W rounded up to a multiple of k*k (any-resolution
 *                   rule); the 1-D modes: see skiparse_mode
 *   sub_h, sub_w    local grid of a subsequence: Hp / k rows, Wp / k columns;
 *                   every subsequence spans all T frames
 *   sub_len_padded  T * sub_h * sub_w slots per subsequence
 *   real_h[p]       real local rows of subsequences with row coordinate p
 *   real_w[q]       real local columns of subsequences with column coordinate q
 *                   The real tokens of subsequence s = p*k + q fill the prefix
 *                   box [0,T) x [0,real_h[p]) x [0,real_w[q]) of its local grid
 *                   (the 1-D modes: s = q, local grid (T, 1, sub_w)).
 *   pairs           computed (real x real, same subsequence) query-key pairs
 *                   of a whole call: sum_s n_s^2 * B * heads; 4 * d * pairs
 *                   is the call's algorithmic FLOP count
 */
typedef struct skiparse_plan {
  int32_t abi;
  int32_t B, T, H, W, heads, d, k, mode;
  int32_t Hp, Wp;
  int32_t sub_h, sub_w;
  int32_t n_sub;
  int32_t reserved0;
  int64_t sub_len_padded;
  int64_t pairs;
  int32_t real_h[SKIPARSE_MAX_K];
  int32_t real_w[SKIPARSE_MAX_K];
} skiparse_plan;

/* Returns SKIPARSE_ABI_VERSION. */
int skiparse_abi_version(void);

/*
 * Fill *plan for tensors of shape (B, T, H, W, heads, d), sparsity factor k
 * (1 <= k <= 8) and pattern mode (token- or group-wise, see the top of this
 * file).  Host only, O(k^2).  Limits: every extent >= 1; T*Hp*Wp < 2^31
 * (Hp, Wp the padded extents); heads*d < 2^31; B*T*H*W*heads*d < 4.6e18.  d outside {64, 128} is accepted here and refused
 * by skiparse_attn_fwd.  Errors: SKIPARSE_EINVAL.
 */
int skiparse_plan_init(skiparse_plan* plan, int32_t B, int32_t T, int32_t H, int32_t W,
                       int32_t heads, int32_t d, int32_t k, int32_t mode);

/*
 * Host index map (the rearrange of the core method, with the any-resolution
 * padding): host_gather[s * sub_len_padded + j] = flat token index
 * (t*H + h)*W + w held by slot j of subsequence s, slots enumerating the
 * padded local grid (T, sub_h, sub_w) row-major, or -1 for a padded slot.
 * host_gather: caller-owned host array of n_sub * sub_len_padded int32.
 * Errors: SKIPARSE_EINVAL.
 */
int skiparse_plan_index_map(const skiparse_plan* plan, int32_t* host_gather);

/*
 * The same map, written on the device by the index function the attention
 * kernels use to gather Q/K/V rows and scatter O rows.  dev_gather: device
 * array of n_sub * sub_len_padded int32.  Errors: SKIPARSE_EINVAL,
 * SKIPARSE_EHIP.
 */
int skiparse_index_map_device(const skiparse_plan* plan, int32_t* dev_gather, hipStream_t stream);

/*
 * Skiparse-2D attention forward (core method + method steps, see the top of
 * this file): for every batch b, head and subsequence s in
 * [sub_begin, sub_begin + sub_count) (sub_count == 0 means all n_sub and
 * then needs sub_begin == 0), each
 * real query token x of s gets
 *     O[x] = sum_y softmax_y(softmax_scale * <Q[x], K[y]>) V[y]
 * over the real tokens y of s.  Rows of O outside the run subsequences are
 * not written.  Padded tokens are never read or written.
 *   dtype             SKIPARSE_F32: q/k/v/o fp32.  SKIPARSE_BF16: q/k/v/o bf16.
 *                     SKIPARSE_FP8_E4M3: q/k/v e4m3 bytes quantized per
 *                     tensor (skiparse_quant_fp8), o bf16.
 *   softmax_scale     <= 0 selects 1/sqrt(d)
 *   dev_descale_qkv   FP8 only: device array of 6 fp32
 *                     {s_q, 1/s_q, s_k, 1/s_k, s_v, 1/s_v}, i.e. the three
 *                     scale pairs skiparse_quant_fp8 writes, back to back;
 *                     NULL otherwise.  Q, K, V stand for code / s.
 *   o                 must not overlap q, k or v.
 * Supported: d in {64, 128} (F32 and BF16), d == 128 (FP8); 1 <= k <= 8.
 * Errors: SKIPARSE_EINVAL, SKIPARSE_EUNSUPPORTED, SKIPARSE_EHIP.
 */
int skiparse_attn_fwd(const skiparse_plan* plan, skiparse_dtype dtype,
                      const void* q, const void* k, const void* v, void* o,
                      float softmax_scale, const float* dev_descale_qkv,
                      int32_t sub_begin, int32_t sub_count, hipStream_t stream);

/*
 * Training forward: skiparse_attn_fwd for SKIPARSE_BF16 that also keeps, for
 * every real query token x of the run subsequences, the natural-log softmax
 * denominator the backward pass needs (the sparse model is fine-tuned and
 * trained with this attention: OSP-Next summary, method steps and
 * reproduction):
 *     lse[(b * T*H*W + x) * heads + head] = log sum_y exp(softmax_scale * <Q[x], K[y]>)
 * over the real tokens y of x's subsequence.  o as in skiparse_attn_fwd.
 *   lse      device fp32, B * T*H*W * heads entries (layout (B, T*H*W, heads)),
 *            4-byte aligned; entries of tokens outside the run subsequences
 *            are not written.  Must not overlap q, k, v or o.
 * Supported: SKIPARSE_BF16, d in {64, 128}.
 * Errors: SKIPARSE_EINVAL, SKIPARSE_EUNSUPPORTED, SKIPARSE_EHIP.
 */
int skiparse_attn_fwd_lse(const skiparse_plan* plan, skiparse_dtype dtype,
                          const void* q, const void* k, const void* v, void* o, float* lse,
                          float softmax_scale, int32_t sub_begin, int32_t sub_count, hipStream_t stream);

/* Workspace bytes skiparse_attn_bwd needs: B * T*H*W * heads * 4 (one fp32
 * per row); 0 for an invalid plan. */
size_t skiparse_attn_bwd_workspace_bytes(const skiparse_plan* plan);

/*
 * Backward pass: the gradients of skiparse_attn_fwd's output with respect to
 * its inputs, for an upstream gradient dout of the same layout as o.  Inside
 * each run subsequence s, with S = softmax_scale * Q K^T over its real tokens,
 * P = softmax(S) by rows (from lse: P = exp(S - lse)), O = P V:
 *     dV = P^T dO,   dS = P * (dO V^T - rowsum(dO * O)),
 *     dQ = softmax_scale * dS K,   dK = softmax_scale * dS^T Q.
 * Rows of dq, dk, dv of the run subsequences' real tokens are written; other
 * rows are not.  Each subsequence is independent, so runs over disjoint
 * subsequence ranges may go to one set of outputs.
 *   q, k, v, o, dout   device bf16 (B, T, H, W, heads, d); o and lse as
 *                      written by skiparse_attn_fwd_lse with the same scale
 *   lse                device fp32 (B, T*H*W, heads), 4-byte aligned
 *   dq, dk, dv         device bf16, same layout as q; must not overlap each
 *                      other, the inputs or the workspace
 *   workspace          device, at least skiparse_attn_bwd_workspace_bytes,
 *                      4-byte aligned, caller-owned scratch (rowsum(dO * O))
 * Supported: SKIPARSE_BF16, d == 128, 1 <= k <= 8.
 * Errors: SKIPARSE_EINVAL, SKIPARSE_EUNSUPPORTED, SKIPARSE_EWORKSPACE,
 * SKIPARSE_EHIP.
 */
int skiparse_attn_bwd(const skiparse_plan* plan, skiparse_dtype dtype,
                      const void* q, const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, void* dq, void* dk, void* dv, float softmax_scale,
                      void* workspace, size_t workspace_bytes,
                      int32_t sub_begin, int32_t sub_count, hipStream_t stream);

/*
 * 8-bit training (OSP-Next summary, 方法步骤详情 method steps and 技术新颖性
 * novelty: the sparse model is trained with per-tensor 8-bit quantization of
 * the forward tensors and of the gradients, each with its own maximum in the
 * scale rule).  Q, K, V and dO arrive as per-tensor e4m3 codes, each with a
 * device pair {scale, 1/scale} as skiparse_quant_fp8 writes it; the gradient
 * dO is quantized by the caller with the gradient maximum it chooses (448, the
 * e4m3 maximum, is this library's reading: the pages give only HiF8 values).
 * Both calls compute on the dequantized tensors Q^ / s_q etc.
 */

/*
 * Training forward on e4m3 inputs: skiparse_attn_fwd with SKIPARSE_FP8_E4M3
 * that also writes the log-sum-exp of the dequantized scores, as
 * skiparse_attn_fwd_lse defines it:
 *     lse[(b * T*H*W + x) * heads + head] = log sum_y exp(softmax_scale * <Q[x], K[y]>),
 *     Q = q8 / s_q, K = k8 / s_k.
 *   q8, k8, v8        device e4m3 codes (B, T, H, W, heads, d), 16-byte aligned
 *   dev_descale_qkv   device 6 fp32: {s_q, 1/s_q, s_k, 1/s_k, s_v, 1/s_v}
 *   o                 device bf16, same layout; lse as in skiparse_attn_fwd_lse.
 *                     Neither may overlap the inputs or each other.
 * Supported: d == 128.  Errors: SKIPARSE_EINVAL, SKIPARSE_EUNSUPPORTED,
 * SKIPARSE_EHIP.
 */
int skiparse_attn_fwd_lse_fp8(const skiparse_plan* plan, const void* q8, const void* k8, const void* v8,
                              const float* dev_descale_qkv, void* o, float* lse, float softmax_scale,
                              int32_t sub_begin, int32_t sub_count, hipStream_t stream);

/*
 * Backward pass on e4m3 inputs: skiparse_attn_bwd's gradients of the
 * dequantized tensors Q = q8 / s_q, K = k8 / s_k, V = v8 / s_v for the
 * dequantized upstream gradient dO = dout8 / s_do.  The products of two
 * coded tensors (S = Q K^T and dP = dO V^T) run on the e4m3 matrix core; P
 * and dS enter the products for dV, dK and dQ as bf16, against the codes.
 *   q8, k8, v8, dev_descale_qkv   as in skiparse_attn_fwd_lse_fp8
 *   o, lse             the bf16 output and log-sum-exp of the forward (for
 *                      example skiparse_attn_fwd_lse_fp8 with the same scale)
 *   dout8              device e4m3 codes of dO, same layout, 16-byte aligned
 *   dev_descale_dout   device 2 fp32: {s_do, 1/s_do}
 *   dq, dk, dv, workspace   as in skiparse_attn_bwd (bf16 gradients); they may
 *                      not overlap each other, the inputs, the scales or lse
 * Supported: d == 128, 1 <= k <= 8.
 * Errors: SKIPARSE_EINVAL, SKIPARSE_EUNSUPPORTED, SKIPARSE_EWORKSPACE,
 * SKIPARSE_EHIP.
 */
int skiparse_attn_bwd_fp8(const skiparse_plan* plan, const void* q8, const void* k8, const void* v8,
                          const float* dev_descale_qkv, const void* o, const void* dout8,
                          const float* dev_descale_dout, const float* lse, void* dq, void* dk, void* dv,
                          float softmax_scale, void* workspace, size_t workspace_bytes, int32_t sub_begin,
                          int32_t sub_count, hipStream_t stream);

/* Workspace bytes skiparse_quant_fp8 needs for numel elements. */
size_t skiparse_quant_fp8_workspace_bytes(int64_t numel);

/*
 * Per-tensor 8-bit quantization with the pages' scale rule
 * scale = fp8_max / (amax + eps), amax = max |x| over the whole tensor, one
 * scale per tensor and no finer blocks (OSP-Next summary, 方法步骤详情 method
 * steps).  The pages' format (HiF8) is replaced by OCP e4m3 with
 * fp8_max = 448.  Every step is IEEE fp32: scale = fp8_max / (amax + eps);
 * y[i] = e4m3(x[i] * scale), rounded to nearest even and saturated to +-448.
 *   x          device, numel elements of x_dtype (SKIPARSE_BF16 or SKIPARSE_F32)
 *   y          device, numel bytes
 *   dev_scale  device, 2 fp32: {scale, 1/scale}
 *   workspace  device, >= skiparse_quant_fp8_workspace_bytes(numel) bytes,
 *              contents need not be initialized; it is overwritten
 * Non-finite inputs are not hidden: a NaN anywhere makes amax, the scale and
 * every code NaN (code 0xFF); an infinity makes the scale 0, so finite
 * elements become signed zeros and the infinities NaN.  Errors:
 * SKIPARSE_EINVAL, SKIPARSE_EWORKSPACE, SKIPARSE_EHIP.
 */
int skiparse_quant_fp8(const void* x, skiparse_dtype x_dtype, int64_t numel, uint8_t* y,
                       float* dev_scale, float fp8_max, float eps,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * skiparse_quant_fp8 for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same quantization, with the per-work-group partial maxima
 * in a scratch array the library holds on each GPU (8 KiB, room for the
 * largest grid, so every numel >= 1 fits; a size past it would be refused
 * with SKIPARSE_EWORKSPACE).  The array lives until the process ends; its
 * device address is looked up once per GPU, on the first call with that GPU
 * current.  Nothing is allocated, freed or synchronized.  Every call on one
 * GPU shares the array: calls that overlap in time on one GPU (different
 * streams, or threads) race and must be serialized by the caller.  Each call
 * writes every partial it reads, so nothing needs clearing between calls.
 * Arguments, results and errors as skiparse_quant_fp8.
 */
int skiparse_quant_fp8_noalloc(const void* x, skiparse_dtype x_dtype, int64_t numel, uint8_t* y,
                               float* dev_scale, float fp8_max, float eps, hipStream_t stream);

/*
 * One attention block of the 8-bit video DiT around the sparse attention.
 * The DiT trains and runs with per-tensor 8-bit quantization,
 * scale = fp8_max / (amax + eps) (OSP-Next summary, 方法步骤详情 method steps;
 * 核心方法 core method: the sparse layers between full-attention ones); the
 * pages name the projections and the rotary position embedding around the
 * attention without defining them, so the block takes their plainest form:
 *     x^ = q8(x)
 *     Q = x^ Wq^T,  K = x^ Wk^T,  V = x^ Wv^T        (e4m3 x e4m3, fp32 accumulation)
 *     Q, K = rope(Q), rope(K)
 *     O = skiparse_attn_fwd(q8(Q), q8(K), q8(V))      (SKIPARSE_FP8_E4M3, all subsequences)
 *     y = q8(O) Wo^T                                   (skiparse_gemm_fp8)
 * q8 is skiparse_quant_fp8 with fp8_max 448, eps 1e-12, one scale per
 * tensor.  rope turns, inside head dimension part a in {t, h, w} of size
 * d_a, the pair (x_2i, x_2i+1) (i counted from the part's start) by the angle
 * pos_a * theta^(-2i / d_a), pos_a the token's frame, row or column; the parts
 * follow each other in the order t, h, w.  The projections' bf16 outputs Q,
 * K, V and the attention's bf16 output O are what gets quantized.
 */

/* Workspace bytes of skiparse_block_fwd_fp8 for this plan (about
 * 10 * B*T*H*W*heads*d); 0 for an invalid plan. */
size_t skiparse_block_workspace_bytes(const skiparse_plan* plan);

/*
 * Forward pass of the block on the stream.
 *   plan          B, T, H, W, heads, d = 128, k and mode of the attention;
 *                 C = heads * d channels per token
 *   x             device bf16 (B, T, H, W, C), 16-byte aligned
 *   w_qkvo        device e4m3 codes of Wq, Wk, Wv, Wo one after the other,
 *                 each (C, C) row-major in (out, in) layout (a linear
 *                 layer's weight), 16-byte aligned
 *   dev_w_scales  device fp32 (4, 2): {scale, 1/scale} of each weight as
 *                 skiparse_quant_fp8 writes them (weight = code / scale)
 *   rope_theta    base of the rotary angles (10000 in the usual form), > 0
 *   rope_dims     {d_t, d_h, d_w}: even, summing to d; NULL or {0, 0, 0} for
 *                 d_h = d_w = 2 * (d / 6), d_t = d - d_h - d_w (44, 42, 42)
 *   y             device bf16 (B, T, H, W, C), 16-byte aligned
 *   workspace     device, >= skiparse_block_workspace_bytes(plan) bytes,
 *                 256-byte aligned; scratch, overwritten
 * y and the workspace must not overlap each other or any input.  Inputs must
 * be finite.  Errors: SKIPARSE_EINVAL, SKIPARSE_EUNSUPPORTED (d != 128),
 * SKIPARSE_EWORKSPACE, SKIPARSE_EHIP (launches before a failing one stay
 * enqueued).
 */
int skiparse_block_fwd_fp8(const skiparse_plan* plan, const void* x, const uint8_t* w_qkvo,
                           const float* dev_w_scales, float rope_theta, const int32_t* rope_dims, void* y,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The block's projection on its own: an e4m3 GEMM with fp32 accumulation and
 * bf16 output (round to nearest even),
 *     y[m][n] = (*dev_sx) * (*dev_sw) * sum_k x[m][k] * w[n][k],
 * x and w holding e4m3 codes; dev_sx and dev_sw are the dequantization
 * factors 1/scale of x and w (the second float skiparse_quant_fp8 writes).
 *   x        device (M, K) row-major, 16-byte aligned
 *   w        device (N, K) row-major ((out, in), a linear layer's weight),
 *            16-byte aligned
 *   y        device bf16 (M, N) row-major, 8-byte aligned; must not overlap
 *            the inputs
 *   M        1 <= M < 2^31;  N, K: multiples of 128 in [128, 65536]
 * Errors: SKIPARSE_EINVAL, SKIPARSE_EUNSUPPORTED (N or K not a multiple of
 * 128), SKIPARSE_EHIP.
 */
int skiparse_gemm_fp8(const uint8_t* x, const uint8_t* w, const float* dev_sx, const float* dev_sw, void* y,
                      int64_t M, int32_t N, int32_t K, hipStream_t stream);

/* Workspace bytes of skiparse_rope_fp8 for this plan; 0 for an invalid plan. */
size_t skiparse_rope_fp8_workspace_bytes(const skiparse_plan* plan);

/*
 * The block's rotary embedding and quantization on their own:
 * y = q8(rope(x)) with the rotation and q8 of skiparse_block_fwd_fp8.  The
 * rotation runs in fp32 from cos/sin rounded to fp32 from float64; the scale
 * comes from max |rope(x)| over the whole tensor.
 *   plan         B, T, H, W, heads and d of x (d a power of two >= 8; k and
 *                mode unused)
 *   x            device bf16 (B, T, H, W, heads, d), 16-byte aligned
 *   rope_theta, rope_dims   as for skiparse_block_fwd_fp8
 *   y            device, B*T*H*W*heads*d e4m3 codes, 16-byte aligned
 *   dev_scale    device, 2 fp32: {scale, 1/scale}
 *   workspace    device, >= skiparse_rope_fp8_workspace_bytes(plan) bytes,
 *                16-byte aligned; scratch, overwritten
 * Errors: SKIPARSE_EINVAL, SKIPARSE_EUNSUPPORTED, SKIPARSE_EWORKSPACE,
 * SKIPARSE_EHIP.
 */
int skiparse_rope_fp8(const skiparse_plan* plan, const void* x, float rope_theta, const int32_t* rope_dims,
                      uint8_t* y, float* dev_scale, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/* Description of the last error on the calling thread ("" if none); valid
 * until the next library call on that thread. */
const char* skiparse_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SKIPARSE_H */
