/*
 * motattn — the joint-attention hot path of the Cosmos 3 Mixture-of-
 * Transformers denoiser forward pass, as hand-written HIP kernels for
 * gfx950 (MI355X), behind a plain C ABI.
 *
 * Sources (pages, by title and section):
 *   "Cosmos 3 方法原理全解" (Cosmos 3 method explained):
 *       §2 packed sequence S = [S_AR, S_DM] and its DM order,
 *       §3 the two MoT rooms and the joint-attention equations O_AR / O_DM,
 *       §5 3D mRoPE coordinates, Δt = 6/TPS, the AR->DM time gap,
 *       §6.3 the flow shift of the noise level,
 *       §7.2 the Euler sampler update,
 *       §12.1 the recommended steps and shift per model and mode.
 *   "NVIDIA 发布 Cosmos 3 系列四个开放权重世界模型" (four new checkpoints),
 *       section "流式生成如何工作": chunk-causal attention against a
 *       key/value cache.
 *
 * Conventions shared by every call:
 *   - Every call returns a mot_status.  Argument checks run on the host
 *     before any launch; on MOT_ERR_INVALID_ARG / MOT_ERR_UNSUPPORTED
 *     nothing was enqueued.  MOT_ERR_HIP reports a failed launch.  Outputs
 *     are undefined after any status other than MOT_OK.
 *   - Device pointers are caller-owned device memory (e.g. torch tensors).
 *     The library allocates no device memory.  Its only global state is a
 *     per-kernel atomic flag recording that the kernel's LDS size attribute
 *     was set (idempotent); calls are thread-safe.  One device per
 *     process is assumed: the flag is not per device.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Device calls only enqueue work on it; they never synchronize.
 *   - bf16 is bfloat16 (1-8-7), stored as 16-bit words; fp32 is IEEE float.
 *   - Element types are passed as int32_t holding a mot_dtype; any other
 *     value is MOT_ERR_INVALID_ARG.
 *   - Strides are in elements.  Device pointers must be 16-byte aligned and
 *     strides multiples of 8 elements (bf16) / 4 elements (fp32) unless a
 *     call says otherwise.
 *   - A device call whose launch would need more than 2^32 - 1 work-items
 *     along one grid dimension (one HIP dispatch) returns
 *     MOT_ERR_UNSUPPORTED; each call states its limit.
 */
#ifndef MOTATTN_H
#define MOTATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOT_ABI_VERSION 2

typedef enum {
  MOT_OK = 0,
  MOT_ERR_INVALID_ARG = 1,
  MOT_ERR_UNSUPPORTED = 2,
  MOT_ERR_HIP = 3
} mot_status;

typedef enum { MOT_BF16 = 0, MOT_FP32 = 1 } mot_dtype;

typedef enum {
  MOT_AR_CAUSAL_DM_FULL = 0, /* method page §3: AR causal, DM reads all */
  MOT_CHUNK_CAUSAL_KV = 1    /* streaming page: prefix + chunk-causal  */
} mot_mask_mode;

typedef enum { MOT_REGION_AR = 0, MOT_REGION_DM_CLEAN = 1, MOT_REGION_DM_NOISY = 2 } mot_region;

typedef enum {
  MOT_KIND_TEXT = 0, MOT_KIND_SPECIAL = 1, MOT_KIND_VIDEO = 2,
  MOT_KIND_AUDIO = 3, MOT_KIND_ACTION = 4, MOT_KIND_PROPRIO = 5
} mot_kind;

/* One group of tokens of the packed sequence (method page §2).
 * n_tokens: TEXT / SPECIAL / AUDIO / ACTION / PROPRIO token count.
 * VIDEO: n_frames latent frames x n_views views x grid_h x grid_w.
 * rate: tokens per second (AUDIO / ACTION) or pixel FPS (VIDEO).
 * frame0: VIDEO absolute first latent frame, or -1 to continue the count.
 * step0: AUDIO / ACTION index of the first token on its time ladder. */
typedef struct {
  int32_t region; /* mot_region */
  int32_t kind;   /* mot_kind   */
  int64_t n_tokens;
  int64_t n_frames;
  int64_t n_views;
  int64_t grid_h;
  int64_t grid_w;
  double rate;
  int64_t frame0;
  int64_t step0;
} mot_segment;

int mot_abi_version(void);
/* Text of a status code; any other value gives "unknown status".  Takes
 * the code as an int32_t, so a C caller may pass any value. */
const char* mot_status_string(int32_t s);

/* Packed-sequence layout (method page §2 and §5), host only.
 * Writes per-token region tags (uint8, mot_region) and (t, h, w) positions
 * (float32 [N][3]) into caller-owned HOST buffers of `capacity` tokens.
 * Text/special tokens: t = h = w = running AR index.  DM origin
 * t0 = n_ar + 15000.  A token k on a ladder of rate TPS sits at
 * t0 + (6.0*k)/TPS evaluated in double and rounded once to float (video
 * uses TPS = FPS/4 and k = absolute latent frame); audio/action h = w = 0;
 * proprio at t0; video h = row, w = view*grid_w + col, ordered
 * frame -> view -> row -> col.
 * Errors: INVALID_ARG for null pointers, bad enums, empty segments, a
 * segment order that breaks §2 (AR, then clean, then noisy; vision, audio,
 * action inside a DM group), token counts or frame / step indices past
 * int64, or N > capacity.  When the segments are valid,
 * *n_tok_out and *n_ar_out receive N and n_ar even if N > capacity, so a
 * first call with capacity 0 (buffers may then be NULL) sizes the buffers;
 * otherwise they receive 0. */
mot_status mot_build_layout(const mot_segment* segs, int32_t n_segs, int64_t capacity,
                            int64_t* n_tok_out, int64_t* n_ar_out,
                            float* pos_thw_host, uint8_t* region_host);

/* Region-split projection (method page §3, §3.2: Reasoner weights for AR
 * rows, Generator weights for DM rows):
 *     Y[r, :] = X[r, :] @ (r < n_ar ? W_ar : W_dm)
 * x: [n_rows, d_in] row-major, dtype in_dt.  w_ar, w_dm: [d_in, d_out]
 * row-major, dtype in_dt.  y: [n_rows, d_out] row-major, dtype out_dt.
 * Used for the fused QKV projection (d_out = 3*H*D, columns [Q|K|V], each
 * [H][D]) and for the output projection.  bf16 inputs accumulate in fp32 on
 * MFMA; a bf16 output is the round-to-nearest-even of the fp32 result.
 * fp32 inputs are computed in fp32.  Supported: in_dt == MOT_BF16 with
 * d_in % 64 == 0 and d_out % 64 == 0, or in_dt == MOT_FP32 (any sizes).
 * 0 <= n_ar <= n_rows; n_rows == 0 is a no-op.  y must not alias x or w.
 * Dispatch limit: bf16 uses one 256-lane workgroup per 128x128 output tile
 * of each room (at most 2^24 - 1 tiles); fp32 uses 16x16 tiles with
 * d_out <= 2^28 - 16. */
mot_status mot_qkv_project(const void* x, const void* w_ar, const void* w_dm, void* y,
                           int64_t n_rows, int64_t n_ar, int64_t d_in, int64_t d_out,
                           int32_t in_dt, int32_t out_dt, void* stream);

typedef enum { MOT_EPI_NONE = 0, MOT_EPI_GELU = 1, MOT_EPI_ADD = 2 } mot_epilogue;

/* The region-split projection with an epilogue on the fp32 result, before
 * the store (method page §3: each room has its own MLP; the layer's
 * residual stream):
 *     MOT_EPI_NONE  y = X W                      (= mot_qkv_project)
 *     MOT_EPI_GELU  y = GELU(X W), GELU(v) = v (1 + erf(v / sqrt 2)) / 2
 *                   (the MLP's first matrix)
 *     MOT_EPI_ADD   y = residual + X W           (the output projection and
 *                   the MLP's second matrix onto the residual stream)
 * with W the row's room as in mot_qkv_project, and the same layouts, types,
 * limits and errors.  residual: [n_rows, d_out] row-major of out_dt, given
 * exactly for MOT_EPI_ADD (else NULL); it may be y itself (each element is
 * read before it is written), but must not otherwise overlap y.
 * INVALID_ARG for an unknown epilogue, a residual missing or given against
 * the epilogue, or a misaligned residual. */
mot_status mot_region_linear(const void* x, const void* w_ar, const void* w_dm, void* y,
                             int64_t n_rows, int64_t n_ar, int64_t d_in, int64_t d_out,
                             int32_t in_dt, int32_t out_dt, int32_t epilogue, const void* residual,
                             void* stream);

/* Region-split LayerNorm (method page §3: each room has its own LayerNorm):
 *     y[r, :] = (x[r, :] - mean_r) / sqrt(var_r + eps) * gamma + beta
 * over the hidden dimension, mean and (biased) variance per row in fp32,
 * with (gamma_ar, beta_ar) for rows r < n_ar and (gamma_dm, beta_dm) for the
 * rest.  x: [n_rows, hidden] row-major of in_dt; y: the same of out_dt (may
 * not overlap x); gamma/beta: device fp32 [hidden].  A room with no rows may
 * pass NULL parameters.  hidden % 8 == 0 and hidden <= 8192; eps > 0.
 * n_rows == 0 is a no-op.  One 64-lane wave per row: n_rows * 64 <=
 * 2^32 - 256.  INVALID_ARG for null or misaligned pointers, bad dtypes,
 * hidden not a multiple of 8, or eps not positive and finite; UNSUPPORTED
 * past the size limits. */
mot_status mot_layernorm_region(const void* x, void* y, int64_t n_rows, int64_t n_ar, int64_t hidden,
                                const float* gamma_ar, const float* beta_ar, const float* gamma_dm,
                                const float* beta_dm, float eps, int32_t in_dt, int32_t out_dt,
                                void* stream);

/* Unified 3D mRoPE (method page §5), in place on x [n_tok][n_heads][head_dim]
 * with element strides tok_stride / head_stride (the last dim contiguous).
 * pos_thw: device float32 [n_tok][3].  Pair k of P = head_dim/2 rotates
 * (x_k, x_{k+P}) by a = pos[axis(k)] * theta^(-2k/head_dim), axis = t for
 * k < sec_t, h for k < sec_t+sec_h, w otherwise.  Angles and their cos/sin
 * are evaluated in fp64, the rotation in fp32, the store rounds RNE.
 * head_dim in {64, 80, 128}; sec_t+sec_h+sec_w == head_dim/2; all >= 0.
 * n_tok == 0 is a no-op.  Dispatch limit: head_dim/8 lanes per token,
 * floor(256 / (head_dim/8)) tokens per 256-lane workgroup, at most
 * 2^24 - 1 workgroups. */
mot_status mrope_apply(void* x, int32_t dt, int64_t n_tok, int32_t n_heads, int32_t head_dim,
                       int64_t tok_stride, int64_t head_stride, const float* pos_thw,
                       int32_t sec_t, int32_t sec_h, int32_t sec_w, float theta, void* stream);

/* Arguments of the masked attention.  Query row r has absolute index
 * i = q0 + r in key space.  Masks (i: query, j: key):
 *   MOT_AR_CAUSAL_DM_FULL (method page §3):  i >= n_ar  or  j <= i
 *   MOT_CHUNK_CAUSAL_KV (streaming page):   j < n_prefix  or
 *        floor((j-n_prefix)/chunk_len) <= floor((i-n_prefix)/chunk_len)
 * q: [nq][H][D], k, v: [nk][H_kv][D], o: [nq][H][D] with the given token
 * and head strides (elements, last dim contiguous).  lse (nullable): fp32
 * [n_batch][H][nq], natural-log sum-exp of the scaled scores.  q_pos / k_pos
 * (nullable, device fp32 [nq][3] / [nk][3]): when set, Q / K are rotated by
 * mRoPE (sec_*, theta) as their tiles are loaded; otherwise they are used as
 * given.  scale == 0 means 1/sqrt(D).  The bf16 kernel keeps D = 80 tiles
 * in the D = 128 layout: its PV products cover dims 0..95 and only dims
 * 0..79 are stored.
 *
 * Grouped key/value heads (method page §12.4 model table, Q / KV heads
 * 16/8, 32/8, 64/8): n_kv_heads = H_kv divides H; query head h reads
 * key/value head h / (H / H_kv).  0 means H_kv = H.
 *
 * Batch (method page §7.2-§7.3: the condition and baseline predictions of a
 * guided sampler step): n_batch independent problems of the same shape and
 * mask in one launch; problem b reads q + b q_bs, k + b k_bs, v + b v_bs
 * and writes o + b o_bs (elements; 0 shares an input, overlapping inputs
 * are allowed, outputs must not overlap) and lse + b H nq.  n_batch 0 means
 * 1, and the batch strides are then ignored.  Positions are shared by the
 * problems. */
typedef struct {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int32_t dt;        /* mot_dtype of q, k, v and o */
  int32_t n_heads;
  int32_t head_dim;  /* 64, 128, or 80 (method page §12.4: Super's hidden 5120 over 64 heads) */
  int32_t mask;      /* mot_mask_mode */
  int64_t nq, nk, q0;
  int64_t q_ts, q_hs, k_ts, k_hs, v_ts, v_hs, o_ts, o_hs;
  int64_t n_ar;
  int64_t n_prefix, chunk_len;
  const float* q_pos;
  const float* k_pos;
  int32_t sec_t, sec_h, sec_w;
  float theta;
  float scale;
  /* ABI version 2 */
  int32_t n_kv_heads; /* 0: n_heads */
  int32_t n_batch;    /* 0: 1 */
  int64_t q_bs, k_bs, v_bs, o_bs;
} mot_attn_args;

/* Flash-style masked attention, O = softmax(mask(Q K^T * scale)) V per head
 * (method page §3 equations; streaming page for the chunk mode).  bf16 runs
 * on MFMA with fp32 online softmax and skips tiles with no allowed pair;
 * fp32 runs on the vector ALUs in fp32.  nq == 0 is a no-op that touches
 * nothing (null pointers allowed; INVALID_ARG for a bad dtype, head count or
 * size, nk < 0 or q0 < 0).  Otherwise requires nk >= q0 + nq
 * in AR mode (every query sees its diagonal), q0 >= n_prefix and chunk_len >=
 * 1 in chunk mode, 0 <= n_ar, n_prefix <= nk, nk >= 1.  bf16 returns
 * MOT_ERR_UNSUPPORTED when k_pos is set (bf16 rotates Q on load only: rotate
 * K beforehand with mrope_apply, which is also the layout a key cache keeps),
 * when nk > 2^31 - 65 or nq > 2^31 - 1, or when a 64-row tile of K or V
 * spans 4 GiB or more (128 * max(k_ts, v_ts) >= 2^32).  INVALID_ARG also
 * for n_kv_heads < 0 or not dividing n_heads, n_batch < 0 or > 65535, and
 * negative or misaligned batch strides.  Dispatch limit: bf16
 * 2 * n_heads * (nq + 512) <= 2^32 - 1; fp32 nq <= 2^32 - 64 and
 * n_heads <= 65535. */
mot_status mot_attention_fwd(const mot_attn_args* args, void* stream);

/* Attention over disjoint key sets merged into attention over their union
 * (the softmax of the method page's §3 equations over all keys):
 *     L = log sum_b exp(L_b),   O = sum_b exp(L_b - L) O_b,   LSE = L.
 * With the batch of mot_attention_fwd over key ranges, this splits one
 * query tile's keys over several workgroups, for calls whose query tiles
 * alone leave the chip idle (the streaming chunk).
 * o_parts: n_parts outputs, part b at o_parts + b * part_stride elements,
 * each [nq][H][D] with token / head strides p_ts / p_hs; lse_parts: fp32
 * [n_parts][H][nq], each part's natural-log LSE as mot_attention_fwd writes
 * it.  o: [nq][H][D] with strides o_ts / o_hs; lse (nullable): fp32 [H][nq]
 * of the union.  Element type dt (bf16 or fp32) for o_parts and o.  In
 * fp32: the max of the parts' LSE, their weights exp(L_b - max), the
 * weighted sum, then division by the weights' sum.  A part whose LSE is
 * -inf for a row (no key) gets weight 0.  1 <= n_parts <= 16; head_dim 64,
 * 80 or 128; nq == 0 is a no-op.  One lane per (row, head, 8 dims): nq * H * D/8
 * <= 2^32 - 256.  INVALID_ARG for null or misaligned pointers, bad strides,
 * counts or dtype; UNSUPPORTED past the dispatch limit. */
mot_status mot_attention_merge(const void* o_parts, const float* lse_parts, int32_t n_parts,
                               int64_t part_stride, int64_t nq, int32_t n_heads, int32_t head_dim,
                               int64_t p_ts, int64_t p_hs, void* o, int64_t o_ts, int64_t o_hs,
                               float* lse, int32_t dt, void* stream);

/* Flow-matching Euler update (method page §7.2), in place:
 *     x[e] = x[e] + (sigma_next - sigma) * v[e],   e < n
 * x: device fp32; v: device bf16 or fp32 (v_dt), contiguous.  The step
 * (sigma_next - sigma) is formed in fp32 and applied with one fused
 * multiply-add.  x_bf16 (nullable): also store bf16(x_new) there (the row
 * block of the next step's packed input).  n == 0 is a no-op. */
mot_status flow_euler_step(float* x, const void* v, int32_t v_dt, int64_t n,
                           float sigma, float sigma_next, void* x_bf16, void* stream);

/* Guided Euler update (method page §7.2: the CFG equation and the Euler
 * step; §7.3: both predictions of a sampler step, then one update), in place:
 *     v    = v_base[e] + guidance * (v_cond[e] - v_base[e])
 *     x[e] = x[e] + (sigma_next - sigma) * v,   e < n
 * in one pass over x, v_cond and v_base.  x: device fp32; v_cond, v_base:
 * device bf16 or fp32 (v_dt), contiguous.  In fp32: the difference, then
 * v = fma(guidance, v_cond - v_base, v_base) and x = fma(sigma_next - sigma,
 * v, x).  x_bf16 (nullable): also store bf16(x_new) there.  n == 0 is a
 * no-op.  INVALID_ARG for a null or misaligned pointer, a bad v_dt or a
 * guidance that is not finite. */
mot_status flow_cfg_euler_step(float* x, const void* v_cond, const void* v_base, int32_t v_dt,
                               int64_t n, float guidance, float sigma, float sigma_next,
                               void* x_bf16, void* stream);

/* Sampler noise levels with the flow shift (method page §6.3 shift map, §7.2
 * sampler loop, §12.1 recommended steps and shift per mode), host only.
 * Writes sigmas_host[k] for k = 0..n_steps into a caller-owned HOST buffer
 * of n_steps + 1 floats: t̄ = (n_steps - k) / n_steps and
 *     sigma_k = shift * t̄ / (1 + (shift - 1) * t̄),
 * evaluated in double, left to right as written, and rounded once to float.
 * sigma_0 = 1 and sigma_n = 0; shift = 1 gives sigma_k = 1 - k/n_steps.
 * Consecutive pairs (sigma_k, sigma_k+1) are the arguments of
 * flow_euler_step.  Errors: INVALID_ARG for n_steps < 1, a null buffer, or a
 * shift outside [2^-20, 2^20] (the pages use 1 to 10; far below that range
 * the denominator cancels). */
mot_status mot_sigma_schedule(int32_t n_steps, double shift, float* sigmas_host);

/* Debug/test helpers: the exact mask and the tile classes the attention
 * kernel uses.  mask_dev: device uint8 [nq][nk] (1 = allowed), nullable.
 * tiles_dev: device uint8 [ceil(nq/bm)][ceil(nk/bn)] (0 empty, 1 partial,
 * 2 full, judged on in-range pairs), nullable.  Only the mask fields of
 * args (mask, nq, nk, q0, n_ar, n_prefix, chunk_len) are read.
 * Dispatch limit: nq * nk (mask) and the tile count each <= 2^32 - 256. */
mot_status mot_mask_materialize(const mot_attn_args* args, uint8_t* mask_dev, int32_t bm,
                                int32_t bn, uint8_t* tiles_dev, void* stream);

/* Host version of the tile classifier, into a HOST buffer of
 * ceil(nq/bm) * ceil(nk/bn) bytes.  INVALID_ARG for null pointers, bm or
 * bn < 1, or mask fields that mot_attention_fwd would reject. */
mot_status mot_tile_classes_host(const mot_attn_args* args, int32_t bm, int32_t bn,
                                 uint8_t* tiles_host);

#ifdef __cplusplus
}
#endif
#endif /* MOTATTN_H */
