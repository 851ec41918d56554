/*
 * attn_int8.h — C ABI of the INT8 FlashAttention-style attention forward for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (see the pages cited on each entry point):
 *   1. per-row symmetric INT8 quantization of Q and K, and of V per tensor or
 *      per row: s = absmax / 127, zero point 0
 *      ("IntAttention: A Fully Integer Attention Pipeline for Efficient Edge
 *      Inference", §2.1 Eq. 3; token-level granularity from
 *      "INT-FlashAttention: Enabling Flash Attention for INT8 Quantization",
 *      abstract);
 *   2. a fused tiled forward: INT8 x INT8 -> INT32 logits, dequantized by
 *      s_Q[i] s_K[j] / sqrt(d) (IntAttention §2.1 and §3.1 Eq. 4; the
 *      row-scale x column-scale form is the vector-wise scheme of
 *      "LLM.int8(): 8-bit Matrix Multiplication for Transformers at Scale",
 *      abstract), an fp32 online softmax over KV tiles (max subtraction as in
 *      IntAttention §2.2; tile-wise fusion as in "FlashAttention-3",
 *      abstract), probabilities quantized to INT8 with multiplier 127
 *      (IntAttention §3.2, the prior-methods scheme), INT8 P.V into INT32 per
 *      tile, and the final rescale O = acc / l with l the row sum of 127 P
 *      (IntAttention §2.1, O ~ s_V P V_hat). The logits are taken in base 2
 *      (the same softmax: e^(S - m) = 2^((S - m) log2 e)).
 *
 * Conventions shared by every entry point:
 *  - Every pointer argument is a DEVICE pointer owned by the caller, except the
 *    output pointers of attn_int8_fwd_schedule and attn_index_softmax_table
 *    (host). The library never allocates, frees, copies between host and
 *    device, or synchronizes.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Work is enqueued on it and the call returns at once.
 *  - All arguments are checked on the host before anything is launched. On any
 *    error nothing is launched, no output is touched, and the status says why.
 *    A launch failure reported by the HIP runtime returns ATTN_ERR_HIP.
 *  - Tensors are dense and row-major with the last dimension innermost:
 *    q [B, H, Lq, d], k and v [B, Hkv, Lkv, d], o [B, H, Lq, d].
 *  - Inputs must be finite; NaN and Inf are outside the contract.
 *  - The functions keep no global mutable state and are reentrant; calls that
 *    run on different streams over disjoint outputs do not interact.
 */
#ifndef ATTN_INT8_H
#define ATTN_INT8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1, /* NULL pointer, bad size, misalignment, bad flag   */
  ATTN_ERR_UNSUPPORTED = 2, /* valid request outside what is implemented       */
  ATTN_ERR_HIP = 3          /* the HIP runtime reported an error at launch     */
} attn_status;

typedef enum { ATTN_F32 = 0, ATTN_F16 = 1 } attn_dtype;

/* V scale granularity: one scale for the tensor, one per token, one per
 * (batch, kv head) (a block granularity), or one per (batch, kv head, channel)
 * (the per-channel granularity); IntAttention §3.3 names both finer schemes as
 * compatible with the method. */
typedef enum {
  ATTN_VSCALE_PER_TENSOR = 0,
  ATTN_VSCALE_PER_TOKEN = 1,
  ATTN_VSCALE_PER_HEAD = 2,
  ATTN_VSCALE_PER_CHANNEL = 3
} attn_vscale;

/*
 * attn_quantize_rows — symmetric INT8 quantization of groups of rows
 * (IntAttention §2.1 Eq. 3; token-level groups from the INT-FlashAttention
 * abstract).
 *
 *   x       [n_rows, n_cols] of x_dt (fp32 or fp16), device, 16-byte aligned.
 *   q       [n_rows, n_cols] int8 output, device, 8-byte aligned.
 *   scales  [n_rows / rows_per_scale] fp32 output, device, 4-byte aligned.
 *   rows_per_scale: consecutive rows sharing one scale. 1 = per token;
 *           n_rows = one scale for the whole tensor; any divisor of n_rows.
 *   n_cols  must be a multiple of 8 (else ATTN_ERR_UNSUPPORTED).
 *
 * For each group with absmax a: if a == 0 then s = 0 and every code is 0;
 * otherwise s = a / 127 and r = 127 / a (each a correctly rounded fp32
 * division) and q = clamp(rne(x * r), -127, 127), where x * r is one rounded
 * fp32 multiply and rne rounds to nearest, ties to even. Codes are in
 * [-127, 127]; -128 is never produced.
 * While the call runs, `scales` is also used as scratch for the group maxima.
 */
attn_status attn_quantize_rows(const void* x, attn_dtype x_dt, int64_t n_rows, int32_t n_cols,
                               int64_t rows_per_scale, int8_t* q, float* scales, void* stream);

/*
 * attn_quantize_cols — symmetric INT8 quantization with one scale per column
 * of each group of rows (the per-channel granularity IntAttention §3.3 names
 * as compatible; the quantizer of §2.1 Eq. 3 applied to each column), e.g.
 * V [B, Hkv, Lkv, d] as n_groups = B * Hkv groups of rows_per_group = Lkv rows
 * gives the [B, Hkv, d] scales of ATTN_VSCALE_PER_CHANNEL.
 *
 *   x       [n_groups, rows_per_group, n_cols] of x_dt (fp32 or fp16), device,
 *           16-byte aligned.
 *   q       same shape, int8 output, device, 8-byte aligned.
 *   scales  [n_groups, n_cols] fp32 output, device, 4-byte aligned.
 *   n_cols  a multiple of 8, at most 2048 (else ATTN_ERR_UNSUPPORTED);
 *           n_groups * n_cols < 2^31 (else ATTN_ERR_UNSUPPORTED).
 *
 * Per (group, column) with absmax a: the same arithmetic as
 * attn_quantize_rows (s = a / 127, r = 127 / a, q = clamp(rne(x * r), +-127);
 * a == 0 gives s = 0 and codes 0). While the call runs, `scales` is also used
 * as scratch for the column maxima.
 */
attn_status attn_quantize_cols(const void* x, attn_dtype x_dt, int64_t n_groups, int64_t rows_per_group,
                               int32_t n_cols, int8_t* q, float* scales, void* stream);

/*
 * attn_quantize_rows_int4 — per-token symmetric 4-bit quantization for INT4
 * Q.K ("INT-FlashAttention: Enabling Flash Attention for INT8 Quantization",
 * abstract: the token-level scheme carries over to INT4; "IntAttention", §2.1
 * related work: Q.K in INT4 with the value path kept at higher precision is
 * nearly lossless). The quantizer of IntAttention §2.1 Eq. 3 with 7 levels
 * per side instead of 127: per row with absmax a, s = a / 7, r = 7 / a
 * (correctly rounded fp32 divisions), code = clamp(rne(x * r), -7, 7); a == 0
 * gives s = 0 and codes 0.
 *
 *   x       [n_rows, n_cols] of x_dt (fp32 or fp16), device, 16-byte aligned.
 *   codes   [n_rows, n_cols] int8 output (values -7..7), 8-byte aligned, or NULL.
 *   packed  [n_rows, n_cols / 2] bytes output, 4-byte aligned, or NULL: per
 *           group of 8 columns, byte j holds code[j] + 8 in its low nibble and
 *           code[j + 4] + 8 in its high nibble (nibble n stands for n - 8).
 *   scales  [n_rows] fp32 output, 4-byte aligned.
 *   At least one of codes and packed. n_cols a multiple of 8, at most 2048
 *   (else ATTN_ERR_UNSUPPORTED).
 */
attn_status attn_quantize_rows_int4(const void* x, attn_dtype x_dt, int64_t n_rows, int32_t n_cols, int8_t* codes,
                                    uint8_t* packed, float* scales, void* stream);

/*
 * attn_quantize_rows_hadamard — per-token quantization of rows first rotated
 * by the normalized Hadamard matrix H / sqrt(n) (n = n_cols), the "incoherent
 * processing" of the "FlashAttention-3" page: an orthogonal rotation of Q and
 * K before low-precision quantization spreads outlier channels over the row,
 * and (Q H)(K H)^T = Q K^T, so the attention is unchanged in exact
 * arithmetic. Rotate Q and K (never V); the forwards then take the codes as
 * usual.
 *
 * The rotation is the fast Walsh-Hadamard transform in fp32 with Sylvester
 * ordering (H[i][j] = (-1)^popcount(i & j)): strides h = 1, 2, 4, ..., n / 2
 * in that order, each pair (a at index e with bit h clear, b at e + h)
 * becoming (a + b, a - b), then every value multiplied by fl32(1 / sqrt(n)).
 * The codes follow attn_quantize_rows (bits = 8, codes in [-127, 127]) or
 * attn_quantize_rows_int4 (bits = 4, codes and / or the packed layout) on
 * the rotated values.
 *
 *   x       [n_rows, n_cols] of x_dt, device, 16-byte aligned.
 *   n_cols  a power of two, 8 .. 2048 (else ATTN_ERR_UNSUPPORTED).
 *   bits    8: codes required, packed must be NULL; 4: codes and / or packed
 *           (else ATTN_ERR_INVALID_ARG).
 *   codes   [n_rows, n_cols] int8 (8-byte aligned), packed [n_rows, n_cols / 2]
 *           (4-byte aligned), scales [n_rows] fp32 (4-byte aligned).
 */
attn_status attn_quantize_rows_hadamard(const void* x, attn_dtype x_dt, int64_t n_rows, int32_t n_cols, int32_t bits,
                                        int8_t* codes, uint8_t* packed, float* scales, void* stream);

/*
 * attn_kv_append_int4 — attn_kv_append for a packed 4-bit K cache (INT4
 * Q.K): the codes and scales of attn_quantize_rows_int4 for the T new tokens
 * x [B, Hkv, T, d] written into rows pos .. pos + T - 1 of every (b, kv head)
 * of cache4 [B, Hkv, L_max, d / 2] (4-byte aligned) and scales
 * [B, Hkv, L_max]; no other row is touched. Argument rules as
 * attn_kv_append.
 */
attn_status attn_kv_append_int4(const void* x, attn_dtype x_dt, int32_t B, int32_t Hkv, int32_t T, int32_t d,
                                uint8_t* cache4, float* scales, int32_t L_max, int32_t pos, void* stream);

/*
 * attn_kv_append — per-token INT8 quantization of new K or V tokens straight
 * into their rows of an INT8 cache (quantize-on-append; the per-token
 * quantizer of IntAttention §2.1 Eq. 3 with the token-level granularity of the
 * INT-FlashAttention abstract, so the cache holds exactly what
 * attn_quantize_rows would produce for the whole tensor).
 *
 *   x       [B, Hkv, T, d] new tokens of x_dt (fp32 or fp16), device,
 *           16-byte aligned.
 *   cache   [B, Hkv, L_max, d] int8, device, 8-byte aligned: rows pos ..
 *           pos + T - 1 of every (b, kv head) receive the codes of the new
 *           tokens; no other row is touched.
 *   scales  [B, Hkv, L_max] fp32, device, 4-byte aligned: the matching
 *           per-token scales.
 *   d       a multiple of 8, at most 2048 (else ATTN_ERR_UNSUPPORTED).
 *   B, Hkv, T, L_max >= 1; 0 <= pos and pos + T <= L_max (else
 *           ATTN_ERR_INVALID_ARG). The cache must have fewer than 2^31 elements.
 *
 * Codes and scales follow attn_quantize_rows with rows_per_scale = 1 exactly.
 * Only per-token scales can be appended (a per-tensor scale would change the
 * rows already in the cache).
 */
attn_status attn_kv_append(const void* x, attn_dtype x_dt, int32_t B, int32_t Hkv, int32_t T, int32_t d,
                           int8_t* cache, float* scales, int32_t L_max, int32_t pos, void* stream);

/*
 * attn_int8_fwd — fused INT8 attention forward (INT-FlashAttention abstract:
 * FlashAttention forward with fully INT8 inputs; formulas as listed at the top
 * of this header).
 *
 *   q    int8 [B, H, Lq, d]      s_q fp32 [B, H, Lq]       (per-token scales)
 *   k    int8 [B, Hkv, Lkv, d]   s_k fp32 [B, Hkv, Lkv]    (per-token scales)
 *   v    int8 [B, Hkv, Lkv, d]   s_v fp32 [1] (ATTN_VSCALE_PER_TENSOR),
 *                                    [B, Hkv, Lkv] (ATTN_VSCALE_PER_TOKEN),
 *                                    [B, Hkv] (ATTN_VSCALE_PER_HEAD) or
 *                                    [B, Hkv, d] (ATTN_VSCALE_PER_CHANNEL)
 *   o    [B, H, Lq, d] of o_dt (fp32 or fp16, rounded to nearest even)
 *   lse  fp32 [B, H, Lq] natural-log log-sum-exp of the scaled logits, or NULL
 *   d    64 or 128 (else ATTN_ERR_UNSUPPORTED)
 *   H % Hkv == 0; query head h reads KV head h / (H / Hkv).
 *   causal 0 or 1. Causal masking is bottom-right aligned: query i sees key j
 *        iff j <= i + (Lkv - Lq); causal requires Lq <= Lkv.
 *   workspace, workspace_bytes: device scratch of at least
 *        attn_int8_fwd_workspace_size(...) bytes, 256-byte aligned (may be
 *        NULL when that size is 0).
 *   int8 tensors and o must be 16-byte aligned, scales 4-byte aligned; each
 *   tensor must have fewer than 2^31 elements.
 *
 * Per row the kernel visits the KV tiles reported by attn_int8_fwd_schedule
 * in ascending order. Each key's logit is taken in base 2,
 * t = (S_int * (s_Q * c)) * s_K[j] in fp32 with c = fl32(log2(e) / sqrt(d)).
 * For tile t with running max m' of t (after the tile) and the exponent bias
 * b = m' - log2(127) in fp32 (moved up one float when m' - b still exceeds
 * log2(127), so that no code passes 127): y = 2^(t - b) = 127 P_tilde,
 * l = alpha l + sum y with alpha = 2^(m_old - m'), P_hat = rne(fl32(y w_j))
 * with w_j = 1 (per-tensor and per-head V) or the fp32 quotient s_V[j] / s_t
 * (per-token V, s_t = the largest s_V of the tile's keys), acc = alpha acc + s_t * (P_hat . V_hat)
 * (s_t = s_V for per-tensor V, the (batch, kv head)'s s_V for per-head V, 1
 * for per-channel V), and finally O = acc / l, channel c multiplied by its
 * scale for per-channel V; lse = ln 2 (m' - log2(127) + log2 l). Because P_hat
 * follows the running max, O depends on the tile size and split points; they
 * are part of the result's definition and are reported by the schedule query.
 */
attn_status attn_int8_fwd(const int8_t* q, const float* s_q, const int8_t* k, const float* s_k,
                          const int8_t* v, const float* s_v, attn_vscale v_mode, void* o,
                          attn_dtype o_dt, float* lse, int32_t B, int32_t H, int32_t Hkv,
                          int32_t Lq, int32_t Lkv, int32_t d, int32_t causal, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * attn_int8_fwd_noalloc — attn_int8_fwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same kernels and results, bit for bit, with no
 * workspace argument. Decode-shaped problems keep their split-KV partials in
 * a static device array of attn_int8_fwd_noalloc_max_scratch() bytes (32 MiB)
 * that the library holds on each GPU it runs on until the process ends; the
 * call allocates and frees nothing (no hipMalloc, no allocating library
 * routine).
 *
 *   Arguments as for attn_int8_fwd, without workspace / workspace_bytes. The
 *   calling thread's current device must be the device of `stream`.
 *   Problems whose attn_int8_fwd_workspace_size(...) exceeds the scratch size
 *   return ATTN_ERR_UNSUPPORTED (nothing launched); every other check and
 *   status is as for attn_int8_fwd.
 *   Every call on one GPU shares that GPU's scratch, and each call's kernels
 *   write every scratch entry they read first (nothing needs clearing), so
 *   calls in stream order are independent; calls that overlap on one GPU
 *   (different streams, or different host threads without ordering) race on
 *   the scratch and their results are undefined.
 */
attn_status attn_int8_fwd_noalloc(const int8_t* q, const float* s_q, const int8_t* k, const float* s_k,
                                  const int8_t* v, const float* s_v, attn_vscale v_mode, void* o,
                                  attn_dtype o_dt, float* lse, int32_t B, int32_t H, int32_t Hkv,
                                  int32_t Lq, int32_t Lkv, int32_t d, int32_t causal, void* stream);

/* attn_int8_fwd_noalloc_max_scratch — bytes of the per-GPU scratch of
 * attn_int8_fwd_noalloc: the largest attn_int8_fwd_workspace_size(...) it
 * accepts. */
size_t attn_int8_fwd_noalloc_max_scratch(void);

/*
 * attn_int8_fwd_qfloat — attn_int8_fwd with the per-token quantization of Q
 * fused into the kernels' Q load (IntAttention §2.1 Eq. 3, token-level as in
 * the INT-FlashAttention abstract): each query row is quantized in the kernel
 * with exactly the arithmetic of attn_quantize_rows (rows_per_scale = 1), so
 * the result is bit-identical to attn_quantize_rows followed by attn_int8_fwd,
 * without the separate pass over Q.
 *
 *   q       [B, H, Lq, d] of q_dt (fp32 or fp16), device, 16-byte aligned.
 *   q_hat   optional int8 output [B, H, Lq, d] (16-byte aligned) receiving the
 *           codes the kernel used, or NULL.
 *   s_q     optional fp32 output [B, H, Lq] (4-byte aligned) receiving the
 *           per-token scales, or NULL.
 *   Every other argument, the schedule and the workspace are as for
 *   attn_int8_fwd.
 */
attn_status attn_int8_fwd_qfloat(const void* q, attn_dtype q_dt, const int8_t* k, const float* s_k,
                                 const int8_t* v, const float* s_v, attn_vscale v_mode, void* o,
                                 attn_dtype o_dt, float* lse, int8_t* q_hat, float* s_q, int32_t B,
                                 int32_t H, int32_t Hkv, int32_t Lq, int32_t Lkv, int32_t d,
                                 int32_t causal, void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * attn_int8_fwd_qfloat_hadamard — attn_int8_fwd_qfloat with each Q row first
 * rotated by the normalized Hadamard matrix inside the kernels' Q load
 * (incoherent processing, "FlashAttention-3" page), with exactly the
 * arithmetic of attn_quantize_rows_hadamard (bits = 8): the codes, scales and
 * O are bit-identical to attn_quantize_rows_hadamard on Q followed by
 * attn_int8_fwd. K must be quantized with the same rotation
 * (attn_quantize_rows_hadamard) for the logits to be Q K^T; V is not rotated.
 * Arguments as attn_int8_fwd_qfloat (q_hat / s_q receive the rotated codes).
 */
attn_status attn_int8_fwd_qfloat_hadamard(const void* q, attn_dtype q_dt, const int8_t* k, const float* s_k,
                                          const int8_t* v, const float* s_v, attn_vscale v_mode, void* o,
                                          attn_dtype o_dt, float* lse, int8_t* q_hat, float* s_q, int32_t B,
                                          int32_t H, int32_t Hkv, int32_t Lq, int32_t Lkv, int32_t d,
                                          int32_t causal, void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_int8_fwd_index_softmax — attn_int8_fwd with IndexSoftmax in place of
 * the exp softmax ("IntAttention: A Fully Integer Attention Pipeline for
 * Efficient Edge Inference", §3.1: the distance to the row max clipped at c
 * and mapped to a 2^b-entry exponential table by
 * idx = floor(distance / c * (2^b - 1)); §3.2: integer row sum and
 * normalisation; §4 ablation: (b, c) = (5, 6.6) recommended), read for
 * per-token Q/K scales and online KV tiles:
 *
 *   table   E_tab[i] = rne(127 exp(-(double)c * i / (2^b - 1)))  (signed
 *           7-bit, as the INT8 products are signed; attn_index_softmax_table)
 *   u_j     = S_int[j] * s_K[j]                                   (fp32)
 *   m_u     = running max of u over the visible keys up to this tile's end
 *   kappa   = (s_Q * (1/sqrt(d))) * ((2^b - 1) / c)               (fp32)
 *   idx_j   = min(floor(max(fma(u_j, -kappa, m_u * kappa), 0)), 2^b - 1)
 *   E_j     = E_tab[idx_j] (0 for masked keys); l = alpha l + sum_j E_j
 *           (the integer tile sum), acc = alpha acc + s_V (E . V_hat)
 *           (INT32 per tile; s_V = 1 for per-channel V), alpha =
 *           exp((m_u,old - m_u,new) s_Q / sqrt(d))
 *   O       = acc / l (channel c times its scale for per-channel V);
 *           lse = m_u s_Q / sqrt(d) + ln(l / 127).
 *
 * The distance is the dequantized logit's (the pages' integer distance with
 * c_int at its exact value c / alpha; with one scale per key an integer
 * distance does not measure logits). Arguments, layouts, schedule, workspace
 * and errors are those of attn_int8_fwd, plus:
 *   lut_bits  b, 1..8 (else ATTN_ERR_INVALID_ARG)
 *   clip      c, finite, in [1e-3, 1e3] (else ATTN_ERR_INVALID_ARG)
 * v_mode ATTN_VSCALE_PER_TOKEN returns ATTN_ERR_UNSUPPORTED (per-key V
 * weights would re-round the table's codes). Inputs whose scaled distances
 * overflow fp32 are outside the contract.
 */
attn_status attn_int8_fwd_index_softmax(const int8_t* q, const float* s_q, const int8_t* k,
                                        const float* s_k, const int8_t* v, const float* s_v,
                                        attn_vscale v_mode, void* o, attn_dtype o_dt, float* lse,
                                        int32_t B, int32_t H, int32_t Hkv, int32_t Lq, int32_t Lkv,
                                        int32_t d, int32_t causal, int32_t lut_bits, float clip,
                                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_index_softmax_table — the table attn_int8_fwd_index_softmax uses for
 * (lut_bits, clip) (IntAttention §3.1-3.2; formula above), written to the
 * HOST buffer table[2^lut_bits]. Same parameter checks; no GPU work.
 */
attn_status attn_index_softmax_table(int32_t lut_bits, float clip, uint8_t* table);

/*
 * attn_int4qk_fwd — the forward with K in packed 4-bit codes (INT4 Q.K; see
 * attn_quantize_rows_int4 for the passages, the codes and the packed layout).
 * gfx950 has no INT4 matrix instruction, so the codes are widened to INT8 for
 * the same INT8 products: S_int = sum_c q_c k_c exactly, everything after it
 * as attn_int8_fwd (the same schedule).
 *
 *   q    int8 [B, H, Lq, d] (codes of attn_quantize_rows_int4, -7..7 for INT4
 *        Q.K; any int8 codes give the exact product)   s_q fp32 [B, H, Lq]
 *   k4   packed [B, Hkv, Lkv, d / 2] bytes, 16-byte aligned   s_k fp32 [B, Hkv, Lkv]
 *   v, s_v, v_mode, o, o_dt, lse, shapes, causal: as attn_int8_fwd.
 *   workspace: at least attn_int4qk_fwd_workspace_size(...) bytes, 256-byte
 *        aligned. Decode-shaped problems read the packed codes directly (the
 *        split-KV partials as for attn_int8_fwd); other shapes first widen K
 *        into the workspace (B Hkv Lkv d bytes) and run the INT8 kernel.
 */
attn_status attn_int4qk_fwd(const int8_t* q, const float* s_q, const uint8_t* k4, const float* s_k, const int8_t* v,
                            const float* s_v, attn_vscale v_mode, void* o, attn_dtype o_dt, float* lse, int32_t B,
                            int32_t H, int32_t Hkv, int32_t Lq, int32_t Lkv, int32_t d, int32_t causal,
                            void* workspace, size_t workspace_bytes, void* stream);

/* attn_int4qk_fwd_workspace_size — bytes of workspace attn_int4qk_fwd needs
 * (0 for invalid problems, which attn_int4qk_fwd then reports). */
size_t attn_int4qk_fwd_workspace_size(int32_t B, int32_t H, int32_t Hkv, int32_t Lq, int32_t Lkv, int32_t d,
                                      int32_t causal);

/*
 * attn_int8_fwd_workspace_size — bytes of device workspace attn_int8_fwd needs
 * for this problem (0 when it needs none; split-KV decode shapes need room for
 * the per-split partial results). Returns 0 for invalid problems as well;
 * attn_int8_fwd then reports the error.
 */
size_t attn_int8_fwd_workspace_size(int32_t B, int32_t H, int32_t Hkv, int32_t Lq, int32_t Lkv,
                                    int32_t d, int32_t causal);

/*
 * attn_int8_fwd_schedule — the schedule facts that change attn_int8_fwd's
 * result (the probability grid follows the running max, so the result depends
 * on where tiles and splits start): *kv_tile = keys per KV tile (tiles start at
 * multiples of it), *kv_split_len = keys per KV split (splits start at
 * multiples of it and are merged by their maxima), or 0 when the KV range is
 * not split. Host pointers. Same argument checks as attn_int8_fwd.
 */
attn_status attn_int8_fwd_schedule(int32_t B, int32_t H, int32_t Hkv, int32_t Lq, int32_t Lkv,
                                   int32_t d, int32_t causal, int32_t* kv_tile,
                                   int32_t* kv_split_len);

/*
 * attn_int8_debug_logits — test entry point: runs the fused prefill kernel
 * itself, in an instance that keeps its grid, its K staging ring and barriers
 * and its INT8 Q.K^T tile code (IntAttention §2.1: INT8 products with INT32
 * accumulation) but writes the exact INT32 logit of every visible pair to
 * s_out [B, H, Lq, Lkv] (int32, device, 16-byte aligned) in place of the
 * softmax and P.V. Pairs masked by the causal rule are not written. Same
 * shape rules as attn_int8_fwd; every shape runs the prefill kernel's tiles.
 */
attn_status attn_int8_debug_logits(const int8_t* q, const int8_t* k, int32_t B, int32_t H,
                                   int32_t Hkv, int32_t Lq, int32_t Lkv, int32_t d, int32_t causal,
                                   int32_t* s_out, void* stream);

/* attn_status_str — static, NUL-terminated description of a status code. */
const char* attn_status_str(attn_status status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_INT8_H */
