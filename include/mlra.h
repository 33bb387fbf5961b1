/*
 * mlra.h - one decode step of attention over a compressed latent KV cache,
 * for AMD Instinct MI355X (gfx950).
 *
 * Methods (pages cited by title and section):
 *   MLA  - multi-head latent attention with weight absorption: the cache holds
 *          one latent row c_t (width d_c) and one RoPE key row k^R_t (width
 *          d_r) per token, shared by all heads ("ML Revisit: Attention",
 *          section Multi-Head Latent Attention; "vllbc02MLA", 苏神思路).
 *   MLRA-n - the multi-branch variant: branch j attends over its own latent
 *          slice [j*d_c/n, (j+1)*d_c/n) plus the shared RoPE key, runs its own
 *          softmax, and the branch outputs are summed ("Multi-Head Low-Rank
 *          Attention", 核心方法 and 方法步骤详情). MLA is n = 1.
 *
 * Per sequence b with cache length L_b and head h the library computes
 *   q_abs  = [alpha_q * tau * W_UK[h] q^N  ||  tau * RoPE(q^R, p_b)]
 *   s_j,t  = q_abs[S_j] . c_t[S_j] + q_abs[rope] . k^R_t          (t < L_b)
 *   o~_j   = sum_t softmax_t(s_j) c_t[S_j]
 *   o      = alpha_kv * W_UV[h]^T concat_j(o~_j)
 * with p_b = L_b - 1 unless a query position is given. L_b = 0 gives o = 0.
 * RoPE rotates consecutive pairs (2i, 2i+1) by p * theta^(-2i/d_r).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers to dense row-major arrays unless
 *     stated; the caller owns them. The library never allocates device memory
 *     and never synchronises: each call only enqueues kernels on `stream`
 *     (a hipStream_t; NULL = the legacy default stream) and results are valid
 *     once that stream's work has completed.
 *   - Host-side validation runs before any launch. On any error nothing is
 *     launched and outputs are left untouched. Errors are reported as status
 *     codes; mlra_last_error_detail() gives text for the calling thread.
 *   - cache_lens values outside [0, max_len] are clamped on the device.
 *   - dtype: MLRA_BF16 means q_nope, q_rope, W_UK, W_UV, the cache and q_abs
 *     are bf16 (accumulation in fp32); MLRA_FP32 means all of them are fp32.
 *     latent_out is always fp32.
 *   - Calls are thread-safe and stateless apart from per-thread error text,
 *     per-thread timing events (mlra_set_kernel_timing) and a per-device
 *     table of device properties filled on first use.
 */
#ifndef MLRA_H_
#define MLRA_H_

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define MLRA_API __attribute__((visibility("default")))
#else
#define MLRA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLRA_OK = 0,
  MLRA_ERR_INVALID_ARG = 1,  /* null pointer, bad size, misaligned pointer or stride */
  MLRA_ERR_UNSUPPORTED = 2,  /* valid but unsupported combination of sizes/dtypes */
  MLRA_ERR_WORKSPACE = 3,    /* workspace missing or smaller than mlra_workspace_size */
  MLRA_ERR_NO_DEVICE = 4,    /* no usable HIP device */
  MLRA_ERR_HIP = 5,          /* a HIP runtime call or kernel launch failed */
  MLRA_ERR_BOUNDS = 6        /* debug build only: a device bounds check failed during the call */
} mlra_status_t;

typedef enum { MLRA_BF16 = 0, MLRA_FP32 = 1 } mlra_dtype_t;

/* Which split-KV decode kernel runs (all compute the same partial state;
 * results agree within the bf16 tolerance). A forced kernel that does not
 * support the configuration gives MLRA_ERR_UNSUPPORTED at the decode call. */
typedef enum {
  MLRA_KERNEL_AUTO = 0,        /* the fastest kernel that supports the shape */
  MLRA_KERNEL_PORTABLE = 1,    /* scalar FMA kernel: any shape, bf16 and fp32 */
  MLRA_KERNEL_HEAD_GROUP = 2,  /* bf16 MFMA, 16 heads per wave over all branches:
                                  d_rope = 64, d_latent in {128, 256, 512},
                                  d_latent / n >= 32, n in {1, 2, 4},
                                  heads in {32, 64, 128} */
  MLRA_KERNEL_BRANCH = 3,      /* bf16 MFMA, one 128-wide branch and 32 heads per
                                  wave: n = 4, d_latent = 512, d_rope = 64,
                                  heads in {64, 128}; and one 128-wide branch
                                  alone (n = 1, d_latent = 128, 128 heads).
                                  fp8 caches: n = 4 at 128 heads */
  MLRA_KERNEL_WIDE = 4         /* fp16 MFMA on the cache converted in LDS, 16 heads
                                  per wave for the scores and 64 latent columns
                                  per wave for P V, across the whole row: n = 1
                                  (MLA), d_latent = 512, d_rope = 64, 128 heads;
                                  bf16 and fp8 caches */
} mlra_kernel_t;
/* The head-group kernel reads bf16 caches only; with an fp8 cache the
 * automatic choice is the branch or wide kernel where they fit, else the
 * portable kernel. */

typedef struct {
  int32_t num_heads;     /* H >= 1 */
  int32_t d_latent;      /* d_c, total latent width (all branches) */
  int32_t d_rope;        /* d_r, even */
  int32_t d_nope;        /* d_n */
  int32_t d_v;           /* value width per head */
  int32_t num_branches;  /* n >= 1, d_latent % n == 0; 1 = MLA */
  float sm_scale;        /* tau; <= 0 selects 1/sqrt(d_nope + d_rope) */
  float alpha_q;         /* multiplies the NoPE score term of every branch */
  float alpha_kv;        /* multiplies the summed branch output */
  float rope_theta;      /* RoPE base, e.g. 10000 */
  mlra_dtype_t dtype;
  int32_t kv_chunk;      /* tokens per split-KV work item; 0 = chosen by the library */
  mlra_kernel_t decode_kernel;  /* MLRA_KERNEL_AUTO unless a kernel is to be forced */
  int32_t q_residue;     /* 0 or 1 (bf16 only): the q_abs rows of mla_absorb_q and
                            mla_decode_attn also carry q~'s rounding residue, see
                            mla_absorb_q; mlra_decode writes it wherever the chosen
                            kernel reads it, and q_residue = 1 also makes the
                            four-branch branch kernel read it (see mla_decode_attn) */
} mlra_config_t;

/* Strided view of the latent cache. Element strides (not bytes). Row t of
 * sequence b is ckv + b*ckv_batch_stride + t*ckv_token_stride (d_latent
 * contiguous elements) and krope + b*krope_batch_stride + t*krope_token_stride
 * (d_rope contiguous elements, stored already rotated at position t). One
 * interleaved buffer of [c_t || k^R_t] rows, two separate buffers, or a branch
 * shard all fit this view.
 *
 * Quantised cache ("MLA多头潜在注意力机制", 9.2 部署注意事项: an 8-bit cache for
 * inference; the pages fix no format, this is the library's reading): with
 * fp8 = 1 the elements are one-byte FP8 E4M3 codes in the OCP 8-bit floating
 * point layout (bias 7, largest finite 448, no infinities) and the values
 * they stand for are c = ckv_scale * e4m3(code) and k^R = krope_scale *
 * e4m3(code): one fp32 scale per cache tensor. Strides are then bytes. Only
 * with cfg->dtype = MLRA_BF16 (queries, weights and outputs stay bf16). The
 * decode calls (mla_decode_attn, mlra_decode, mlra_decode_noalloc) accept it;
 * mlra_prefill returns MLRA_ERR_UNSUPPORTED. With fp8 = 0 the scales are
 * ignored and the elements have cfg->dtype.
 *
 * Value range: the MFMA decode kernels (head-group, branch, wide) keep each
 * work item's partial latent output, a weighted mean of cache rows, in fp16
 * between the decode and the merge, and the wide kernel and the fp16 modes
 * convert the cache itself to fp16; latent values beyond fp16's range
 * (|c| > 65504) saturate there. The portable kernel has no such limit. */
typedef struct {
  const void* ckv;
  const void* krope;
  int64_t ckv_batch_stride, ckv_token_stride;
  int64_t krope_batch_stride, krope_token_stride;
  const int32_t* cache_lens;  /* device [B] */
  int32_t max_len;            /* rows allocated per sequence */
  int32_t fp8;                /* 0: elements of cfg->dtype; 1: FP8 E4M3 codes */
  float ckv_scale;            /* fp8: finite, in [2^-32, 2^32] */
  float krope_scale;          /* fp8: finite, in [2^-32, 2^32] */
} mlra_cache_t;

/* Bytes of workspace that mla_decode_attn and mlra_decode need for this
 * configuration, batch size and max_len. Host-only; launches nothing. */
MLRA_API mlra_status_t mlra_workspace_size(const mlra_config_t* cfg, int32_t batch, int32_t max_len,
                                  size_t* bytes);

/* Step 1, query-side absorption ("Multi-Head Low-Rank Attention", 方法步骤详情
 * step 1; "ML Revisit: Attention", Multi-Head Latent Attention: W_UK moves
 * into the query; RoPE on the query part only, "从MHA到MLA" 3.2).
 *   q_nope [B][H][d_nope], q_rope [B][H][d_rope] (unrotated), dtype cfg->dtype
 *   q_pos  [B] int32 query positions, or NULL to use cache_lens[b] - 1
 *   cache_lens [B] int32 (read only when q_pos is NULL)
 *   w_uk   [H][d_latent][d_nope]
 *   q_abs  out [B][H][d_latent + d_rope], dtype cfg->dtype; with
 *          cfg->q_residue = 1 (bf16), rows of d_latent + d_rope + d_latent:
 *          q~ rounded to bf16, rho, then the residue bf16(q~ - bf16(q~)), so
 *          that the two bf16 parts carry q~ to about 16 significant bits.
 * All branches are covered at once: branch j's absorbed query is the slice
 * S_j of q_abs. A query rounded to one bf16 moves a score by about 2^-9 of
 * its spread; at MLA's scales on the pages (alpha_q = sqrt(7168 / 512)) that
 * alone moves output rows by up to ~1.3e-2 in relative L2, which the residue
 * removes. */
MLRA_API mlra_status_t mla_absorb_q(const mlra_config_t* cfg, int32_t batch, const void* q_nope,
                           const void* q_rope, const int32_t* q_pos, const int32_t* cache_lens,
                           const void* w_uk, void* q_abs, void* stream);

/* Step 2, MQA-style decode over [C_KV || K_RoPE] in latent space, one online
 * softmax per branch, split over the token axis and merged
 * ("Multi-Head Low-Rank Attention", 方法步骤详情 step 2; "vllbc02MLA",
 * 苏神思路: decoding works like MQA).
 *   q_abs      [B][H][d_latent + d_rope] from mla_absorb_q (rows of
 *              d_latent + d_rope + d_latent with cfg->q_residue = 1; the
 *              residue enters the scores of every kernel. The four-branch
 *              branch kernel (MLRA-4 at 128 heads) then runs in fp16: q~
 *              from both parts, the tiles converted in LDS, P in fp16, about
 *              19% more time on a bf16 cache and ~1.4e-3 instead of
 *              ~7.4e-3 worst-row error; it always does with an fp8 cache)
 *   cache      strided cache view (16-byte aligned bases and byte strides
 *              that are multiples of 16). With an fp8 cache the call first
 *              writes q~ * ckv_scale and rho * krope_scale into the workspace
 *              (the caller's q_abs is not changed) and latent_out is the
 *              latent of the dequantised cache (times ckv_scale).
 *   workspace  device buffer of at least mlra_workspace_size() bytes
 *   latent_out out [B][H][d_latent] fp32 = concat_j o~_j (branch-normalised) */
MLRA_API mlra_status_t mla_decode_attn(const mlra_config_t* cfg, int32_t batch, const void* q_abs,
                              const mlra_cache_t* cache, void* workspace, size_t ws_bytes,
                              float* latent_out, void* stream);

/* The split-KV decode kernel that mla_decode_attn and mlra_decode run for
 * this configuration, batch and cache view (cfg->decode_kernel resolved).
 * Host-only; launches nothing and needs no device. Same validation as
 * mla_decode_attn for cfg and cache; MLRA_ERR_UNSUPPORTED when a forced
 * kernel does not support the configuration. */
MLRA_API mlra_status_t mlra_select_decode_kernel(const mlra_config_t* cfg, int32_t batch,
                                                 const mlra_cache_t* cache, mlra_kernel_t* kernel);

/* Step 3, output up-projection and branch sum ("Multi-Head Low-Rank
 * Attention", 方法步骤详情 step 3 and the sum over branches in 核心方法):
 *   out[b][h] = alpha_kv * W_UV[h]^T latent_out[b][h]
 *   latent_out [B][H][d_latent] fp32, w_uv [H][d_latent][d_v] (cfg->dtype),
 *   out [B][H][d_v] in out_dtype. */
MLRA_API mlra_status_t mla_out_proj(const mlra_config_t* cfg, int32_t batch, const float* latent_out,
                           const void* w_uv, void* out, mlra_dtype_t out_dtype, void* stream);

/* The whole decode step (steps 1-3) for MLRA with `num_branches` branches
 * (overrides cfg->num_branches; 1 = MLA). Intermediates live in the workspace.
 * Arguments as for the three calls above. With an fp8 cache the scales are
 * folded into the absorbed query (q~ * ckv_scale, rho * krope_scale) and the
 * output scale (alpha_kv * ckv_scale): the result is the decode of the
 * dequantised cache. */
MLRA_API mlra_status_t mlra_decode(const mlra_config_t* cfg, int32_t num_branches, int32_t batch,
                          const void* q_nope, const void* q_rope, const int32_t* q_pos,
                          const void* w_uk, const void* w_uv, const mlra_cache_t* cache,
                          void* workspace, size_t ws_bytes, void* out, mlra_dtype_t out_dtype,
                          void* stream);

/* mlra_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same kernels and results, with the workspace taken from
 * a 128 MiB device array that the library holds on each GPU it runs on
 * (allocated when the library's code object loads there, freed when the
 * process ends) instead of a caller's buffer. It calls no allocator.
 * Arguments and validation as for mlra_decode. The workspace is sized for
 * the work items this call's plan makes (at 128 heads, d_latent 512, B = 16
 * and kv_chunk = 0 about 47 MB for MLRA-4 and 80 MB for MLA, whatever the
 * cache length); a call that needs more returns MLRA_ERR_WORKSPACE and
 * launches nothing. Every call on
 * one GPU shares that GPU's array, so calls that overlap in time on one GPU
 * (different streams or threads) race and give undefined results;
 * serialise them. */
MLRA_API mlra_status_t mlra_decode_noalloc(const mlra_config_t* cfg, int32_t num_branches,
                                           int32_t batch, const void* q_nope, const void* q_rope,
                                           const int32_t* q_pos, const void* w_uk,
                                           const void* w_uv, const mlra_cache_t* cache, void* out,
                                           mlra_dtype_t out_dtype, void* stream);

/* The step before the decode: append one token per sequence to the latent
 * cache ("vllbc02MLA", 猛猿大佬思路: the projected row splits into the
 * compressed latent, which is RMS-normalised, and the decoupled RoPE key,
 * rotated by the token's position; "从MHA到MLA" 3.2: the new latent is written
 * at that position; "MLA多头潜在注意力机制" 3: only these two are cached).
 *
 *   new_rows   device [batch][d_latent + d_rope] fp32, row-major: the new
 *              token's latent c (pre-normalisation) then its RoPE key k^R
 *              (unrotated), as produced by the model's down-projection.
 *   gain       device [d_latent] fp32 RMSNorm weight, or NULL for all ones.
 *   eps        RMSNorm epsilon (> 0 or 0; DeepSeek uses 1e-6).
 *   ckv, krope device cache buffers of cfg->dtype, written through the same
 *              element strides as mlra_cache_t (krope unused when d_rope = 0).
 *   cache_lens device [batch] int32, read and updated in place.
 *   max_len    rows each sequence can hold.
 *
 * For each sequence b with p = max(L_b, 0) < max_len: row p of the latent
 * cache gets c / sqrt(mean(c^2) + eps) * gain, row p of the RoPE cache gets
 * RoPE(k^R, p) (pairs (2i, 2i+1), angle p * theta^(-2i/d_rope), angle in
 * double precision), both rounded to the cache dtype (bf16: RNE), then L_b
 * becomes p + 1. A sequence with L_b >= max_len is left unchanged, since that
 * cannot be reported without a synchronisation. The next decode call's
 * query then sits at position p, the new token. Sizes, pointer and stride
 * checks as for the decode: INVALID_ARG on a NULL pointer or a negative
 * size or stride, UNSUPPORTED for sizes beyond the decode's limits. Enqueued
 * on `stream`; nothing is allocated. */
MLRA_API mlra_status_t mlra_cache_append(const mlra_config_t* cfg, int32_t batch,
                                         const float* new_rows, const float* gain, float eps,
                                         void* ckv, void* krope, int64_t ckv_batch_stride,
                                         int64_t ckv_token_stride, int64_t krope_batch_stride,
                                         int64_t krope_token_stride, int32_t* cache_lens,
                                         int32_t max_len, void* stream);

/* mlra_cache_append into an fp8 cache (see mlra_cache_t): the same row values
 * as mlra_cache_append, each stored as the FP8 E4M3 code nearest value /
 * scale (fp32 division, round to nearest with ties to the even mantissa,
 * saturating at +-448; ckv_scale for the latent, krope_scale for the RoPE
 * key). ckv and krope are byte buffers, strides in bytes (= elements).
 * Needs cfg->dtype = MLRA_BF16; scales finite and in [2^-32, 2^32]. */
MLRA_API mlra_status_t mlra_cache_append_fp8(const mlra_config_t* cfg, int32_t batch,
                                             const float* new_rows, const float* gain, float eps,
                                             void* ckv, void* krope, int64_t ckv_batch_stride,
                                             int64_t ckv_token_stride,
                                             int64_t krope_batch_stride,
                                             int64_t krope_token_stride, int32_t* cache_lens,
                                             int32_t max_len, float ckv_scale, float krope_scale,
                                             void* stream);

/* Causal prefill over the cache ("MLA多头潜在注意力机制" 3.3: a key after the
 * query's position is masked; "Multi-Head Low-Rank Attention", 核心方法 and
 * 方法步骤详情: one softmax per branch, outputs summed with alpha_kv). For every
 * position t < L_b of every sequence b, out[b][t][h] is what mlra_decode
 * returns for sequence b when its cache holds the rows 0..t and its query
 * sits at position t: the same absorbed form, with t's own query.
 *
 *   q_nope  device [batch][max_len][H][d_nope], q_rope [batch][max_len][H][d_rope]
 *           (unrotated; position t of sequence b is row (b, t)), bf16.
 *   w_uk, w_uv  as for mlra_decode.
 *   cache   as for mlra_decode; rows 0..L_b-1 hold the prompt (for example
 *           from mlra_cache_append); its max_len is the prompt length T.
 *   out     device [batch][max_len][H][d_v], out_dtype; rows t >= L_b get 0.
 *
 * One kernel: absorption, attention and the W_UV projection stay on chip, so
 * no workspace is needed. For MLA (num_branches = 1) use mla_prefill, the
 * unabsorbed form. Supported: bf16 MLRA-4 at d_latent 512, d_rope 64,
 * d_nope 128, d_v 128, per-sequence byte ranges below 2^31 and
 * batch * max_len <= 2^22 rows, else UNSUPPORTED; argument checks as for
 * mlra_decode. With d_c' = d_nope = d_v this absorbed form costs the same
 * multiply-adds as the unabsorbed one. Enqueued on `stream`; nothing is
 * allocated. */
MLRA_API mlra_status_t mlra_prefill(const mlra_config_t* cfg, int32_t num_branches, int32_t batch,
                                    const void* q_nope, const void* q_rope, const void* w_uk,
                                    const void* w_uv, const mlra_cache_t* cache, void* out,
                                    mlra_dtype_t out_dtype, void* stream);

/* Causal prefill of MLA (one branch) in the unabsorbed, multi-head form
 * ("vllbc02MLA", 苏神思路: the prefill is compute-bound and runs as ordinary
 * multi-head attention over keys and values up-projected from the latent;
 * the decode uses the absorbed form; "MLA多头潜在注意力机制" 3.2-3.3: K^N =
 * C W_UK and V = C W_UV per head, the RoPE key shared by all heads, a key
 * after the query's position masked). For every position t < L_b of every
 * sequence b, out[b][t][h] is what mlra_decode with num_branches = 1 returns
 * for sequence b when its cache holds the rows 0..t and its query sits at
 * position t; rows t >= L_b get 0. cfg->num_branches is ignored (1).
 *
 *   q_nope, q_rope, w_uk, w_uv, cache, out   as for mlra_prefill
 *   workspace  device buffer of at least mla_prefill_workspace_size() bytes
 *              (256-byte aligned): K^N (pre-scaled by alpha_q tau log2 e),
 *              V [B][H][T][128] and k^R [B][T][64] as fp16, T = max_len;
 *              2 * B * T * (256 H + 64) bytes.
 *
 * Two kernels: the up-projection (a bf16 MFMA GEMM per head) and causal
 * flash attention on fp16 MFMA. Supported: bf16, d_latent 512, d_rope 64,
 * d_nope 128, d_v 128, any head count, per-sequence byte ranges below 2^31
 * and batch * max_len <= 2^22 rows, else UNSUPPORTED; an fp8 cache is
 * UNSUPPORTED. Enqueued on `stream`; nothing is allocated. The timing events
 * of mlra_set_kernel_timing bracket the attention kernel. */
MLRA_API mlra_status_t mla_prefill_workspace_size(const mlra_config_t* cfg, int32_t batch,
                                                  int32_t max_len, size_t* bytes);
MLRA_API mlra_status_t mla_prefill(const mlra_config_t* cfg, int32_t batch, const void* q_nope,
                                   const void* q_rope, const void* w_uk, const void* w_uv,
                                   const mlra_cache_t* cache, void* workspace, size_t ws_bytes,
                                   void* out, mlra_dtype_t out_dtype, void* stream);

/* Instrumentation: when both are non-NULL hipEvent_t handles (created by the
 * caller, owned by the caller, valid until timing is stopped), every later
 * call made on this thread has the split-KV decode dispatch (mlra_decode,
 * mla_decode_attn) or the causal attention dispatch (mlra_prefill) stamp
 * `before` when it starts and `after` when it ends (hipExtLaunchKernel), so that
 * hipEventElapsedTime gives that kernel's duration and the stream carries no
 * extra packets. Pass NULL, NULL to stop. Giving only one is INVALID_ARG. */
MLRA_API mlra_status_t mlra_set_kernel_timing(void* before, void* after);

/* Static text for a status code. */
MLRA_API const char* mlra_status_string(mlra_status_t status);

/* Detail of the last error on the calling thread ("" if none). */
MLRA_API const char* mlra_last_error_detail(void);

/* 1 in the debug build (libmlra_debug.so, built with MLRA_DEBUG_BOUNDS), 0 in
 * the release build. The debug build checks, on the device, the indices the
 * split-KV plan hands the decode and merge kernels (sequence, token range,
 * partial-state slot, work item, the merge's slot range); a failed check is
 * recorded without stopping the kernel, and mlra_decode,
 * mlra_decode_noalloc and mla_decode_attn then wait for their stream and
 * return MLRA_ERR_BOUNDS (the detail names the check). Takes no arguments and
 * has no failure mode. */
MLRA_API int mlra_bounds_checks(void);

#ifdef __cplusplus
}
#endif

#endif /* MLRA_H_ */
