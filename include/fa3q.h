/*
 * fa3q.h -- C ABI of libfa3q, the FA3 per-head INT8 path for AMD Instinct MI355X (gfx950).
 *
 * The library computes the data-parallel hot path of "FA3" per-head INT8
 * quantisation of MLA attention activations and the decode-phase attention
 * that reads the quantised K cache:
 *
 *   1. fa3q_calibrate_perhead  -- per-head Recall Window of one calibration batch
 *   2. fa3q_accumulate_minmax  -- running min/max across calibration batches
 *      (fa3q_init_minmax sets the running state to its identity first)
 *   3. fa3q_qparams            -- symmetric per-head scale = abs_max / 127
 *   4. fa3q_quantize_k         -- non-RoPE part of K -> INT8 codes, RoPE part kept in bf16
 *   5. fa3q_decode_attn        -- single-query attention over INT8 K-nope + bf16 K-rope + bf16 V
 *   6. fa3q_decode_append_attn -- one decode step: append the new token to the cache in place
 *      (K-nope quantised as in 4), then attention over ragged per-sequence lengths
 *   7. fa3q_decode_attn_qkv8   -- attention with Q (non-RoPE part), K-nope and V all INT8
 *   8. fa3q_quantize_asym      -- non-RoPE part of K -> asymmetric INT8 codes with a scale and
 *      an offset per (head, dim); RoPE part kept in bf16
 *   9. fa3q_decode_attn_asym   -- attention as in 5 over the asymmetric K-nope cache of 8
 *  10. fa3q_calibrate_batches  -- 1 and 2 over several calibration batches in one call
 *  11. fa3q_decode_latent      -- attention of every head of a sequence over one shared-latent
 *      (absorbed MLA) cache: INT8 latent (one scale) + bf16 RoPE part, on the matrix cores
 *  12. fa3q_fake_quant         -- quantise and dequantise (the codes of 4 turned back into bf16),
 *      in place or into a second buffer
 *  13. fa3q_decode_paged_attn  -- 6 over a paged cache: pools of fixed-size pages and a block
 *      table per sequence
 *  14. fa3q_decode_attn_noalloc -- 5 with the library's own static scratch instead of a
 *      caller workspace (for callers that cannot allocate device memory)
 *  15. fa3q_calibrate_ex, fa3q_quantize_k_ex, fa3q_decode_attn_ex, fa3q_decode_append_attn_ex
 *      -- 10, 4, 5 and 6 with a dtype (bf16 or float16 activations, K-rope and V) and a
 *      layout ((B,H,S,D) or (B,S,H,D)) argument
 *
 * Sources, cited by page title and section:
 *   [MS] msModelSlim documentation, "FA3量化：Flash Attention 3激活量化算法说明"
 *        (FA3 quantization: Flash Attention 3 activation quantization algorithm),
 *        sections 原理 -> 算法流程 (algorithm flow) and 适用要求 (requirements).
 *   [MI] MindIE LLM user guide, "FA3 quantization", overview paragraph.
 *   [MT] MindIE Turbo documentation, "Attention量化" (attention quantization),
 *        tables 1 and 2 (q/k/v scale and offset of shape [head_num, head_dim]).
 *
 * Conventions shared by every entry point:
 *   - Every pointer is a DEVICE pointer owned by the caller; the library never
 *     allocates, frees or retains memory and keeps no state between calls (the one
 *     exception is the static scratch array of fa3q_decode_attn_noalloc).
 *   - `stream` is a hipStream_t passed as void*; NULL means the default stream.
 *     Calls only enqueue work on `stream`; they never synchronise.
 *   - Arguments are validated on the host BEFORE anything is enqueued: a
 *     non-zero status means nothing was launched and no output was touched.
 *     Validation makes no HIP call, so it works on a host without a GPU.
 *   - FA3Q_ERR_HIP means a launch was rejected by the HIP runtime; earlier
 *     kernels of the same call may already be enqueued.
 *   - bf16 tensors are passed as their raw 16-bit patterns (uint16_t).
 *   - Inputs must be finite; for NaN/Inf inputs the outputs are unspecified
 *     (the kernels stay inside their buffers for any input bits).
 *   - Outputs must not overlap inputs, except the in/out running statistics and
 *     fa3q_fake_quant's in-place form.
 *   - Concurrent calls on different streams are safe if they use distinct
 *     output and workspace buffers.
 */
#ifndef FA3Q_H_
#define FA3Q_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa3q_status {
  FA3Q_OK = 0,
  FA3Q_ERR_NULL = 1,        /* a required pointer is NULL */
  FA3Q_ERR_DTYPE = 2,       /* unknown dtype code */
  FA3Q_ERR_SHAPE = 3,       /* a size is <= 0, too large, or not a multiple the kernels need */
  FA3Q_ERR_RATIO = 4,       /* ratio not in (0, 1], or int(ratio*N) < 1 */
  FA3Q_ERR_ALIGN = 5,       /* a pointer is not aligned as documented */
  FA3Q_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than the *_workspace_bytes query */
  FA3Q_ERR_HIP = 7,         /* the HIP runtime rejected a launch */
  FA3Q_ERR_UNSUPPORTED = 8, /* valid arguments outside what this build handles (see each call) */
  FA3Q_ERR_ALIAS = 9,       /* an output partly overlaps an input (where exact aliasing is allowed) */
  FA3Q_ERR_SCRATCH = 10,    /* the call needs more scratch than the library's static array holds */
  FA3Q_ERR_LAYOUT = 11      /* unknown layout code */
} fa3q_status;

typedef enum fa3q_dtype {
  FA3Q_F32 = 0,  /* IEEE binary32 */
  FA3Q_BF16 = 1, /* bfloat16, raw 16-bit patterns */
  FA3Q_F16 = 2   /* IEEE binary16, raw 16-bit patterns */
} fa3q_dtype;

/*
 * Memory order of a 4-D activation or cache tensor (row-major in the order named):
 * (batch, head, token, dim) with each head's tokens contiguous, or (batch, token, head, dim)
 * with each token's heads contiguous.  Calls without a layout argument take FA3Q_BHSD.
 */
typedef enum fa3q_layout {
  FA3Q_BHSD = 0,
  FA3Q_BSHD = 1
} fa3q_layout;

/*
 * Signatures take and return plain `int` for statuses, dtype and layout codes: the values
 * are those of fa3q_status, fa3q_dtype and fa3q_layout, but C leaves the integer type
 * behind an enum to the compiler, while `int` has one fixed width for every caller
 * (ctypes, other FFIs).
 */

/* Human-readable name of a status code (static string, never NULL). */
const char* fa3q_status_string(int status);

/* ABI version: (major << 16) | minor. */
int fa3q_version(void);

/* ------------------------------------------------------------------------ */
/* 1. Recall Window calibration                                              */
/* ------------------------------------------------------------------------ */

/*
 * Largest number of windows K = N - int(ratio*N) + 1 that the streaming tail selection
 * (on-chip lists of the K smallest and K largest values) takes for `dtype`.  16-bit input
 * (bf16, float16) with a larger K, with heads of at least 2^20 values or in the FA3Q_BSHD
 * layout takes the histogram path; float32 input with a larger K, or in the FA3Q_BSHD layout
 * with rows of D values that are not a power of two, takes the collect-and-sort path.  Both
 * handle every K.  0 for an unknown dtype.
 */
int64_t fa3q_calibrate_max_windows(int dtype);

/*
 * Device workspace fa3q_calibrate_perhead needs for these arguments, in bytes
 * (0 when the arguments are invalid).  Depends only on the arguments.
 */
size_t fa3q_calibrate_workspace_bytes(int dtype, int64_t B, int64_t H, int64_t S, int64_t D,
                                      double ratio);

/*
 * [MS] 算法流程, per-head statistics and Recall Window.  For one calibration
 * batch x of shape (B, H, S, D), row-major, every head h gathers its
 * N = B*S*D values x[:, h, :, :] (grouped per head, not a raw reshape),
 * sorts them (float32 total order, -0.0 before +0.0), sets
 * t = int(ratio*N) (ratio*N rounded as an IEEE double, then truncated toward
 * zero) and among the windows [s[i], s[i+t-1]], i = 0 .. N-t inclusive, picks
 * the one whose float32 length s[i+t-1] - s[i] is smallest, the smallest i on
 * ties.  Writes win_min[h] = s[i*] and win_max[h] = s[i*+t-1] (float32 values
 * of the input; exact, no rounding).
 *
 *   x          device, dtype FA3Q_F32, FA3Q_BF16 or FA3Q_F16, (B,H,S,D) contiguous,
 *              16-byte aligned.
 *   B,H,S,D    > 0; S*D must be a multiple of 8 (16-bit dtypes) or 4 (f32); N = B*S*D < 2^32.
 *   ratio      in (0, 1]; t = int(ratio*N) must be >= 1.
 *   win_min,
 *   win_max    device float32 [H], 4-byte aligned.
 *   workspace  device, 256-byte aligned, >= fa3q_calibrate_workspace_bytes(...).
 *
 * No sort: one pass over x.  Only the K = N-t+1 smallest and K largest values of a
 * head can bound a window; while K <= fa3q_calibrate_max_windows(dtype) and a head holds
 * fewer than 2^20 values, the kernels select those two tails on chip.  A 16-bit head is
 * otherwise counted into a 65536-bin histogram (its sorted order exactly) and the window
 * found from the counts, for every K.  A float32 head with K above
 * fa3q_calibrate_max_windows(FA3Q_F32) is counted by its values' leading 16 bits, which
 * fixes the leading bits at ranks K-1 and t-1; a second pass collects every value at or
 * below the first or at or above the second (both tails, M >= K values), a radix sort
 * orders them and the K windows are scanned.  That path's workspace holds two lists of N
 * keys per head (twice the size of a float32 batch), reused by every batch of a call.
 * No valid ratio is refused.
 */
int fa3q_calibrate_perhead(const void* x, int dtype, int64_t B, int64_t H, int64_t S, int64_t D,
                           double ratio, float* win_min, float* win_max, void* workspace,
                           size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* 2. Cross-batch accumulation                                               */
/* ------------------------------------------------------------------------ */

/*
 * Sets run_min[h] = +inf and run_max[h] = -inf, the identities of the running
 * min/max of [MS] 算法流程 (cross-batch accumulation).  float32 [H] device
 * arrays, 4-byte aligned, H > 0.
 */
int fa3q_init_minmax(float* run_min, float* run_max, int64_t H, void* stream);

/*
 * [MS] 算法流程, cross-batch accumulation: in place,
 *   run_min[h] = min(run_min[h], cur_min[h]),  run_max[h] = max(run_max[h], cur_max[h])
 * under the float32 total order (-0.0 < +0.0).  All float32 [H] device arrays,
 * 4-byte aligned; cur_* may be the win_min/win_max of fa3q_calibrate_perhead.
 */
int fa3q_accumulate_minmax(float* run_min, float* run_max, const float* cur_min,
                           const float* cur_max, int64_t H, void* stream);

/* ------------------------------------------------------------------------ */
/* 3. Symmetric per-head scale                                               */
/* ------------------------------------------------------------------------ */

/*
 * [MS] 算法流程, quantisation parameters, and 适用要求 (INT8 symmetric only):
 *   scale[h] = max(|run_min[h]|, |run_max[h]|) / 127
 * as one correctly rounded float32 division.  float32 [H] device arrays,
 * 4-byte aligned.  A head whose range is {0} gets scale 0.
 */
int fa3q_qparams(const float* run_min, const float* run_max, float* scale, int64_t H,
                 void* stream);

/* ------------------------------------------------------------------------ */
/* 4. K-cache quantisation                                                   */
/* ------------------------------------------------------------------------ */

/*
 * [MI] overview: only the non-RoPE part of K is quantised to 8 bits, per
 * head; the RoPE part of K is not quantised.  For every row (b, h, s) of the
 * bf16 tensor k (B, H, S, Dn+Dr):
 *   k_nope_q[b,h,s,d] = clamp(round_half_even(fl32(x / scale[h])), -127, 127),  d < Dn
 *                       with x the float32 value of k[b,h,s,d]; 0 when scale[h] == 0
 *   k_rope[b,h,s,j]   = k[b,h,s,Dn+j] bit for bit,  j < Dr
 *
 *   k         device bf16 (B,H,S,Dn+Dr) contiguous, 16-byte aligned.
 *   scale     device float32 [H] (from fa3q_qparams), 4-byte aligned.
 *   k_nope_q  device int8 (B,H,S,Dn) contiguous, 16-byte aligned.
 *   k_rope    device bf16 (B,H,S,Dr) contiguous, 16-byte aligned; may be NULL iff Dr == 0.
 *   B,H,S > 0; Dn > 0 multiple of 16, Dn <= 4096; Dr >= 0 multiple of 8, Dr <= 2048.
 */
int fa3q_quantize_k(const uint16_t* k, const float* scale, int8_t* k_nope_q, uint16_t* k_rope,
                    int64_t B, int64_t H, int64_t S, int64_t Dn, int64_t Dr, void* stream);

/* ------------------------------------------------------------------------ */
/* 5. Decode attention over the quantised cache                             */
/* ------------------------------------------------------------------------ */

/*
 * Device workspace fa3q_decode_attn needs, in bytes (0 when none is needed or
 * the arguments are invalid); the call splits long caches over several
 * workgroups per (b, h) and merges their partial softmax states here.
 */
size_t fa3q_decode_attn_workspace_bytes(int64_t B, int64_t H, int64_t T, int64_t Dv);

/*
 * [MI] overview: the INT8 K-nope cache serves the decode-phase attention
 * operator.  One query token per (b, h) attends to all T cached tokens:
 *   s_t   = sm_scale * ( scale[h] * sum_{d<Dn} q[b,h,d] * k_nope_q[b,h,t,d]
 *                        + sum_{j<Dr} q[b,h,Dn+j] * k_rope[b,h,t,j] )
 *   out[b,h,:] = sum_t softmax(s)_t * v[b,h,t,:]
 * i.e. attention over the cache dequantised per head (scale[h] * code).
 * Arithmetic is float32 (exact int8/bf16 widening, float32 accumulation).
 *
 *   q          device bf16 (B,H,Dn+Dr) contiguous, 16-byte aligned.
 *   k_nope_q   device int8 (B,H,T,Dn), 16-byte aligned.
 *   scale      device float32 [H].
 *   k_rope     device bf16 (B,H,T,Dr), 16-byte aligned; may be NULL iff Dr == 0.
 *   v          device bf16 (B,H,T,Dv), 16-byte aligned.
 *   out        device float32 (B,H,Dv), 16-byte aligned.
 *   B,H,T > 0; Dn in {16,32,...,1024} with Dn/16 a power of two or Dn/16 <= 64;
 *   Dr a multiple of 8 with Dr/8 <= 64; at least one of Dn, Dr > 0 with
 *   Dn % 16 == 0; Dv a power of two in [8, 512].
 *   workspace  device, 256-byte aligned, >= fa3q_decode_attn_workspace_bytes(B,H,T,Dv);
 *              may be NULL when that query returns 0.
 */
int fa3q_decode_attn(const uint16_t* q, const int8_t* k_nope_q, const float* scale,
                     const uint16_t* k_rope, const uint16_t* v, int64_t B, int64_t H,
                     int64_t T, int64_t Dn, int64_t Dr, int64_t Dv, float sm_scale, float* out,
                     void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* 6. Decode step: append the new token, attend over ragged lengths         */
/* ------------------------------------------------------------------------ */

/*
 * [MI] overview: the INT8 K-nope cache is written during decode as each new
 * token's K is produced, and read by the same step's attention.  The cache has
 * room for T tokens per (b, h); sequence b holds kv_len[b] of them.
 *
 * With k_new != NULL (append): for every (b, h), with p = kv_len[b],
 *   k_nope_q[b,h,p,:] = clamp(round_half_even(fl32(k_new[b,h,d] / scale[h])), -127, 127)
 *                       for d < Dn (0 for a head with scale 0), exactly as fa3q_quantize_k,
 *   k_rope[b,h,p,:]   = k_new[b,h,Dn:Dn+Dr]   (bit copy),
 *   v[b,h,p,:]        = v_new[b,h,:]          (bit copy),
 * then out[b,h,:] is the attention of fa3q_decode_attn over tokens 0..p
 * (p + 1 tokens).  Requires 0 <= kv_len[b] <= T-1.
 * With k_new == NULL (and v_new == NULL): attention over tokens
 * 0..kv_len[b]-1, nothing is written to the cache.  Requires 1 <= kv_len[b] <= T.
 *
 *   q, scale, out, T, Dn, Dr, Dv, sm_scale, workspace: as fa3q_decode_attn
 *              (the workspace query takes the capacity T).
 *   k_new      device bf16 (B,H,Dn+Dr), 16-byte aligned, or NULL.
 *   v_new      device bf16 (B,H,Dv), 16-byte aligned; NULL exactly when k_new is.
 *   k_nope_q, k_rope, v  the cache as in fa3q_decode_attn with capacity T; written
 *              in place at position kv_len[b] when appending.
 *   kv_len     device int32 [B], 4-byte aligned; read on the device, not changed.
 *              Lengths outside the required range are clamped into it (the kernels
 *              never leave the cache); the caller advances kv_len after the step.
 * Ownership and errors as for every call; the cache rows written are only
 * those at position kv_len[b].
 */
int fa3q_decode_append_attn(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                            const float* scale, int8_t* k_nope_q, uint16_t* k_rope, uint16_t* v,
                            const int32_t* kv_len, int64_t B, int64_t H, int64_t T, int64_t Dn,
                            int64_t Dr, int64_t Dv, float sm_scale, float* out, void* workspace,
                            size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* 7. Decode attention with Q, K and V per-head INT8                        */
/* ------------------------------------------------------------------------ */

/*
 * [MS] 简介 (overview): FA3 quantises the Q, K and V activations of attention
 * to INT8, one scale per head.  Q's non-RoPE part and all of V get per-head
 * codes from fa3q_quantize_k (V as a (B,H,T,Dv) tensor with Dr = 0, Q as a
 * (B,H,1,Dn+Dr) tensor whose RoPE part comes back as bf16), each with its own
 * calibrated scale; K-nope is the cache of fa3q_quantize_k.  For every (b, h):
 *   s_t   = sm_scale * ( scale_q[h] * scale_k[h] * sum_{d<Dn} qc[b,h,d] * kc[b,h,t,d]
 *                        + sum_{j<Dr} q_rope[b,h,j] * k_rope[b,h,t,j] )
 *   out[b,h,:] = scale_v[h] * sum_t softmax(s)_t * vc[b,h,t,:]
 * i.e. fa3q_decode_attn's attention over the dequantised Q, K and V.  The
 * integer dot product is exact (int32); the rest is float32.
 *
 *   q_nope_q   device int8 (B,H,Dn), 16-byte aligned.
 *   q_rope     device bf16 (B,H,Dr), 16-byte aligned; may be NULL iff Dr == 0.
 *   scale_q, scale_k, scale_v  device float32 [H], 4-byte aligned.
 *   k_nope_q, k_rope  the cache as in fa3q_decode_attn.
 *   v_q        device int8 (B,H,T,Dv), 16-byte aligned.
 *   out, T, Dn, Dr, sm_scale, workspace  as fa3q_decode_attn (same workspace query).
 *   Dv a power of two in [16, 512].
 */
int fa3q_decode_attn_qkv8(const int8_t* q_nope_q, const uint16_t* q_rope, const float* scale_q,
                          const int8_t* k_nope_q, const float* scale_k, const uint16_t* k_rope,
                          const int8_t* v_q, const float* scale_v, int64_t B, int64_t H, int64_t T,
                          int64_t Dn, int64_t Dr, int64_t Dv, float sm_scale, float* out, void* workspace,
                          size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* 8. Asymmetric K-cache quantisation with per-(head, dim) tables            */
/* ------------------------------------------------------------------------ */

/*
 * [MT] tables 1 and 2: the K activation carries a scale and an offset per
 * (head, dim), as float16 (table 1) or bfloat16 (table 2).  The page gives no
 * formula or calibration for them; they are caller inputs, and the code is the
 * plain asymmetric INT8 one.  For every row (b, h, s) of k (B, H, S, Dn+Dr):
 *   k_nope_q[b,h,s,d] = clamp(round_half_even(fl32(fl32(x / sc) + of)), -128, 127),  d < Dn
 *                       with x the float32 value of k[b,h,s,d], sc = scale[h,d] and
 *                       of = offset[h,d] widened exactly to float32, the division
 *                       correctly rounded; 0 when sc == 0
 *   k_rope[b,h,s,j]   = k[b,h,s,Dn+j] bit for bit,  j < Dr
 * A code stands for the value (code - of) * sc.
 *
 *   k             device bf16 (B,H,S,Dn+Dr) contiguous, 16-byte aligned.
 *   scale, offset device [H][Dn] row-major, dtype params_dtype (FA3Q_BF16 or
 *                 FA3Q_F16), 16-byte aligned; finite.
 *   k_nope_q      device int8 (B,H,S,Dn) contiguous, 16-byte aligned.
 *   k_rope        device bf16 (B,H,S,Dr) contiguous, 16-byte aligned; may be NULL iff Dr == 0.
 *   B,H,S > 0; Dn > 0 multiple of 16, Dn <= 4096; Dr >= 0 multiple of 8, Dr <= 2048.
 *   FA3Q_ERR_DTYPE for any other params_dtype.
 */
int fa3q_quantize_asym(const uint16_t* k, const uint16_t* scale, const uint16_t* offset,
                       int params_dtype, int8_t* k_nope_q, uint16_t* k_rope, int64_t B, int64_t H,
                       int64_t S, int64_t Dn, int64_t Dr, void* stream);

/* ------------------------------------------------------------------------ */
/* 9. Decode attention over the asymmetric K cache                           */
/* ------------------------------------------------------------------------ */

/*
 * [MI] overview and [MT] tables 1 and 2: fa3q_decode_attn's attention with the
 * K-nope cache of fa3q_quantize_asym dequantised per (head, dim):
 *   s_t   = sm_scale * ( sum_{d<Dn} q[b,h,d] * (k_nope_q[b,h,t,d] - offset[h,d]) * scale[h,d]
 *                        + sum_{j<Dr} q[b,h,Dn+j] * k_rope[b,h,t,j] )
 *   out[b,h,:] = sum_t softmax(s)_t * v[b,h,t,:]
 * Arithmetic is float32: q[b,h,d] * scale[h,d] is formed once per (b, h) and
 * the offset term sum_d q[b,h,d] * scale[h,d] * offset[h,d] is one constant
 * per (b, h) subtracted from every score.
 *
 *   scale, offset, params_dtype  as fa3q_quantize_asym.
 *   q, k_nope_q, k_rope, v, out, B, H, T, Dn, Dr, Dv, sm_scale, workspace
 *                 as fa3q_decode_attn (same workspace query).
 */
int fa3q_decode_attn_asym(const uint16_t* q, const int8_t* k_nope_q, const uint16_t* scale,
                          const uint16_t* offset, int params_dtype, const uint16_t* k_rope,
                          const uint16_t* v, int64_t B, int64_t H, int64_t T, int64_t Dn, int64_t Dr,
                          int64_t Dv, float sm_scale, float* out, void* workspace,
                          size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* 10. Several calibration batches: windows and running min/max in one call  */
/* ------------------------------------------------------------------------ */

/*
 * Device workspace fa3q_calibrate_batches needs, in bytes (0 when the arguments are
 * invalid, nb outside 1..16 included).
 */
size_t fa3q_calibrate_batches_workspace_bytes(int dtype, int64_t nb, int64_t B, int64_t H, int64_t S,
                                              int64_t D, double ratio);

/*
 * [MS] 算法流程: each calibration batch gives per-head Recall Windows, and the running
 * statistics keep the smallest window minimum and largest window maximum over batches.
 * For batches b = 0 .. nb-1 of the same shape, in order:
 *   (win_min[b], win_max[b]) = fa3q_calibrate_perhead(xs[b], ...)   (bit for bit)
 *   run_min = min(run_min, win_min[b]), run_max = max(run_max, win_max[b])  (as fa3q_accumulate_minmax)
 * with run_min/run_max starting at (+inf, -inf) when init != 0 (fa3q_init_minmax), at
 * their current contents otherwise.  The batches share each launch (one sample, one
 * streaming pass over all of them, one merge and one accumulation), except on the float32
 * collect-and-sort path, which takes them one after the other through one workspace region.
 *
 *   xs         HOST array of nb device pointers, each as x of fa3q_calibrate_perhead
 *              (dtype, (B,H,S,D) contiguous, 16-byte aligned); read during the call only.
 *   nb         1 .. 16.
 *   run_min, run_max  device float32 [H], 4-byte aligned, in/out.
 *   win_min, win_max  device float32 [nb][H], 4-byte aligned, or both NULL (the windows
 *              then live in the workspace only).
 *   workspace  device, 256-byte aligned, >= fa3q_calibrate_batches_workspace_bytes(...).
 *   Other arguments and errors as fa3q_calibrate_perhead; FA3Q_ERR_SHAPE for nb out of range.
 */
int fa3q_calibrate_batches(const void* const* xs, int64_t nb, int dtype, int64_t B, int64_t H, int64_t S, int64_t D,
                           double ratio, float* run_min, float* run_max, int init, float* win_min, float* win_max,
                           void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* 11. Decode attention over a shared-latent (absorbed MLA) cache            */
/* ------------------------------------------------------------------------ */

/*
 * Device workspace fa3q_decode_latent needs, in bytes (0 when none is needed or
 * the arguments are invalid): the partial results of the token splits when there
 * are several, and with H >= 128 one word per 32 heads and split (a split whose
 * scores outgrow the reference its first tile set is marked there and recomputed
 * by a second launch).  No state is kept between calls.
 */
size_t fa3q_decode_latent_workspace_bytes(int64_t B, int64_t H, int64_t T, int64_t Dl);

/*
 * [MI] overview: in MLA attention only the non-RoPE part of K goes to 8 bits,
 * the RoPE part stays floating point.  With the up-projections absorbed into the
 * query, all H query heads of sequence b read the same cache rows: a latent
 * c[b,t,:] of Dl INT8 codes with ONE scale s (the per-head method of 1-4 run
 * with one head, e.g. fa3q_quantize_k on a (B,1,T,Dl+Dr) tensor) and Dr bf16
 * RoPE features k_rope[b,t,:].  For q[b,h,:] = [q_abs (Dl) | q_rope (Dr)]:
 *   s_t        = sm_scale * ( s * sum_{d<Dl} q_abs[d] * c[b,t,d] + sum_{j<Dr} q_rope[j] * k_rope[b,t,j] )
 *   out[b,h,:] = s * sum_t softmax(s)_t * c[b,t,:]        (latent-space output)
 * Both products run on the matrix cores with float32 accumulation; the softmax
 * weights enter the second product as two bf16 terms (hi + lo), so each weight
 * carries a relative error below 2^-17.
 *
 *   q          device bf16 (B,H,Dl+Dr) contiguous, 16-byte aligned.
 *   c_q        device int8 (B,T,Dl) contiguous, 16-byte aligned.
 *   scale      device float32 [1], 4-byte aligned.
 *   k_rope     device bf16 (B,T,Dr), 16-byte aligned; may be NULL iff Dr == 0.
 *   out        device float32 (B,H,Dl), 16-byte aligned.
 *   B,H,T > 0; Dl in {128, 256, 512}; Dr in {0, 32, 64}.
 *   workspace  device, 256-byte aligned, >= fa3q_decode_latent_workspace_bytes(B,H,T,Dl);
 *              may be NULL when that query returns 0.
 */
int fa3q_decode_latent(const uint16_t* q, const int8_t* c_q, const float* scale, const uint16_t* k_rope,
                       int64_t B, int64_t H, int64_t T, int64_t Dl, int64_t Dr, float sm_scale, float* out,
                       void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* 12. Fake quantisation (quantise, then dequantise)                         */
/* ------------------------------------------------------------------------ */

/*
 * [MS] 原理 -> 伪量化部署阶段 (fake-quantisation deployment stage): after calibration
 * the per-head min/max give the symmetric parameters and the observer is replaced by
 * a quantisation node.  The page gives no formula for that node; this is the plain
 * reading, the code of fa3q_quantize_k turned back into a bf16 value:
 *   y[b,h,s,d]    = round_half_even_to_bf16( fl32( code * scale[h] ) ),  d < Dn
 *                   code = clamp(round_half_even(fl32(x / scale[h])), -127, 127) exactly as
 *                   fa3q_quantize_k (0 when scale[h] == 0, so y = +0)
 *   y[b,h,s,Dn+j] = x[b,h,s,Dn+j] bit for bit,  j < Dr
 * The float32 product is correctly rounded, then rounded once more to bf16.
 *
 *   x       device bf16 (B,H,S,Dn+Dr) contiguous, 16-byte aligned.
 *   scale   device float32 [H], 4-byte aligned; finite and >= 0 (as fa3q_qparams gives).
 *   y       device bf16 (B,H,S,Dn+Dr) contiguous, 16-byte aligned: either x itself (in
 *           place; the RoPE part is then neither read nor written) or memory that does
 *           not overlap x (FA3Q_ERR_ALIAS otherwise).
 *   B,H,S > 0; Dn > 0 multiple of 16, Dn <= 4096; Dr >= 0 multiple of 8, Dr <= 2048.
 */
int fa3q_fake_quant(const uint16_t* x, const float* scale, uint16_t* y, int64_t B, int64_t H, int64_t S,
                    int64_t Dn, int64_t Dr, void* stream);

/* ------------------------------------------------------------------------ */
/* 13. Decode step over a paged cache                                        */
/* ------------------------------------------------------------------------ */

/*
 * [MI] overview (the INT8 K-nope cache written and read in the decode phase), as
 * fa3q_decode_append_attn, with the cache held in pages.  The pages leave the cache
 * layout open; here each of the three caches is a pool of num_pages pages of
 * page_size (P) tokens, laid out (num_pages, H, P, .) row-major, so one page of one
 * head is P contiguous rows.  Logical token t of sequence b lives in physical page
 * block_table[b][t / P] at row t % P.  With T = max_pages * P, the call computes what
 * fa3q_decode_append_attn computes on the (B,H,T,.) cache that the block table
 * describes, and the append writes the new rows into the page that holds position
 * kv_len[b].
 *
 *   q, k_new, v_new, scale, sm_scale, out: as fa3q_decode_append_attn.
 *   k_nope_pool  device int8 (num_pages,H,P,Dn), 16-byte aligned.
 *   k_rope_pool  device bf16 (num_pages,H,P,Dr), 16-byte aligned; may be NULL iff Dr == 0.
 *   v_pool       device bf16 (num_pages,H,P,Dv), 16-byte aligned.
 *   block_table  device int32 [B][max_pages], 4-byte aligned; read on the device.  Only
 *                the entries of pages that hold tokens 0..kv_len[b] (with an append) or
 *                0..kv_len[b]-1 are read.  Entries outside [0, num_pages) are clamped
 *                into it, so the kernels never leave a pool.  A page shared by several
 *                sequences is read by each; appending into a shared page writes it for all.
 *   kv_len       device int32 [B], as fa3q_decode_append_attn with capacity T.
 *   page_size    a power of two, 16 .. 65536.  num_pages, max_pages > 0.
 *   workspace    device, 256-byte aligned, >= fa3q_decode_attn_workspace_bytes(B,H,T,Dv)
 *                with T = max_pages * page_size; may be NULL when that query returns 0.
 * Ownership and errors as for every call; the only rows written are those of position
 * kv_len[b] when appending.
 */
int fa3q_decode_paged_attn(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new, const float* scale,
                           int8_t* k_nope_pool, uint16_t* k_rope_pool, uint16_t* v_pool,
                           const int32_t* block_table, const int32_t* kv_len, int64_t B, int64_t H,
                           int64_t num_pages, int64_t page_size, int64_t max_pages, int64_t Dn, int64_t Dr,
                           int64_t Dv, float sm_scale, float* out, void* workspace, size_t workspace_bytes,
                           void* stream);

/* ------------------------------------------------------------------------ */
/* 14. Decode attention with no workspace argument                           */
/* ------------------------------------------------------------------------ */

/* Bytes of the static device array fa3q_decode_attn_noalloc uses as its scratch. */
#define FA3Q_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): fa3q_decode_attn with the same
 * arguments minus the workspace, and the same result bit for bit (same kernels, same
 * split plan).  The split softmax states go to a file-scope device array of
 * FA3Q_NOALLOC_SCRATCH_BYTES bytes that the library holds on every GPU it runs on until
 * the process ends; the call allocates and frees nothing.
 *
 *   Arguments as fa3q_decode_attn.  Calls whose fa3q_decode_attn_workspace_bytes(B,H,T,Dv)
 *   exceeds FA3Q_NOALLOC_SCRATCH_BYTES return FA3Q_ERR_SCRATCH before anything is
 *   enqueued (e.g. B*H = 1024, Dv = 128 is accepted up to T = 65536).  The first call on
 *   a device that needs scratch looks up that device's copy of the array (a HIP call);
 *   FA3Q_ERR_HIP if that fails.
 *   All calls on one GPU share its array: calls that overlap in time on one GPU (on
 *   different streams, or from different threads without ordering) race and give
 *   undefined results.  Calls ordered on one stream are safe.
 */
int fa3q_decode_attn_noalloc(const uint16_t* q, const int8_t* k_nope_q, const float* scale,
                             const uint16_t* k_rope, const uint16_t* v, int64_t B, int64_t H,
                             int64_t T, int64_t Dn, int64_t Dr, int64_t Dv, float sm_scale,
                             float* out, void* stream);

/* ------------------------------------------------------------------------ */
/* 15. float16 input and (B,S,H,D) layouts                                   */
/* ------------------------------------------------------------------------ */

/*
 * [MT] tables 1 and 2 list float16 as well as bfloat16 variants of attention quantisation,
 * and [MI] overview places the quantised K cache in the decode-phase KV cache, whose
 * serving layouts keep either each head's tokens or each token's heads contiguous.  These
 * entry points are 10, 4, 5 and 6 with the activation dtype and the tensor layout as
 * arguments; every result is that of the (B,H,S,D) call on the tensors re-laid out, bit for
 * bit where 4, 5, 6 and 10 are exact, and the same float32 arithmetic otherwise.
 *
 *   dtype   FA3Q_BF16 or FA3Q_F16 for every 16-bit tensor of the call (activations, K,
 *           K-rope, q, V, k_new, v_new; calibration also takes FA3Q_F32); else
 *           FA3Q_ERR_DTYPE.  Codes stay int8, scales and outputs float32.
 *   layout  FA3Q_BHSD or FA3Q_BSHD for every 4-D tensor of the call (activations x, K, the
 *           codes, K-rope and V of the cache); else FA3Q_ERR_LAYOUT.  Tensors of one token
 *           per (b, h) -- q, k_new, v_new, out -- are (B,H,.) in both layouts.
 */

/* Workspace of fa3q_calibrate_ex (0 when the arguments are invalid, nb outside 1..16 included). */
size_t fa3q_calibrate_ex_workspace_bytes(int dtype, int layout, int64_t nb, int64_t B, int64_t H,
                                         int64_t S, int64_t D, double ratio);

/*
 * fa3q_calibrate_batches with a layout: head h of batch b gathers x[b][:, h, :, :] (BHSD)
 * or x[b][:, :, h, :] (BSHD), N = B*S*D values, and the windows and running statistics
 * follow.  run_min and run_max may both be NULL when win_min and win_max are given: the
 * windows are then written and no running statistics kept (fa3q_calibrate_perhead for
 * nb = 1).  BSHD rows of D values must be a multiple of 8 (16-bit) or 4 (float32) values;
 * (B,S,H,D) 16-bit input always takes the histogram path; float32 input takes the tail lists
 * when D is a power of two and K is within fa3q_calibrate_max_windows(FA3Q_F32), the
 * collect-and-sort path otherwise (any K; see fa3q_calibrate_perhead).  Other arguments,
 * alignment and errors as fa3q_calibrate_batches.
 */
int fa3q_calibrate_ex(const void* const* xs, int64_t nb, int dtype, int layout, int64_t B, int64_t H,
                      int64_t S, int64_t D, double ratio, float* run_min, float* run_max, int init,
                      float* win_min, float* win_max, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * fa3q_quantize_k with a dtype and a layout: k is (B,H,S,Dn+Dr) or (B,S,H,Dn+Dr) of dtype,
 * k_nope_q and k_rope have k's layout (rows of Dn int8 codes and Dr values of dtype), and
 * row (b, h, s) is quantised with scale[h] exactly as fa3q_quantize_k does (the quotient of
 * the float32 value of the float16 or bf16 input).  Sizes, alignment and errors as
 * fa3q_quantize_k.
 */
int fa3q_quantize_k_ex(const void* k, const float* scale, int8_t* k_nope_q, void* k_rope, int dtype,
                       int layout, int64_t B, int64_t H, int64_t S, int64_t Dn, int64_t Dr,
                       void* stream);

/*
 * fa3q_decode_attn with a dtype and a layout: q (B,H,Dn+Dr), k_rope and v of dtype; the
 * cache tensors k_nope_q, k_rope and v are (B,H,T,.) or (B,T,H,.).  Workspace query,
 * sizes, alignment and errors as fa3q_decode_attn.
 */
int fa3q_decode_attn_ex(const void* q, const int8_t* k_nope_q, const float* scale, const void* k_rope,
                        const void* v, int dtype, int layout, int64_t B, int64_t H, int64_t T,
                        int64_t Dn, int64_t Dr, int64_t Dv, float sm_scale, float* out,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa3q_decode_append_attn with a dtype and a layout: q, k_new (B,H,Dn+Dr) and v_new
 * (B,H,Dv) of dtype; the cache (capacity T) in the layout, written in place at token
 * kv_len[b] when appending (the new K-nope row quantised as fa3q_quantize_k_ex would).
 * Other arguments and errors as fa3q_decode_append_attn.
 */
int fa3q_decode_append_attn_ex(const void* q, const void* k_new, const void* v_new, const float* scale,
                               int8_t* k_nope_q, void* k_rope, void* v, const int32_t* kv_len,
                               int dtype, int layout, int64_t B, int64_t H, int64_t T, int64_t Dn,
                               int64_t Dr, int64_t Dv, float sm_scale, float* out, void* workspace,
                               size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA3Q_H_ */
