/*
 * qkrope.h -- C ABI of the fused QK-RMSNorm + RoPE (+ V) attention prologue for AMD Instinct
 * MI355X (gfx950).
 *
 * The library computes, in one kernel launch per call, the attention prologue of video and
 * diffusion transformers as two API pages define it:
 *
 *   [table form] vLLM-Omni "vllm_omni.diffusion.layers.fused_qk_norm_rope", module contract and
 *       the fused_qk_norm_rope signature: Q/K RMSNorm with [head_dim] weights, then RoPE from a
 *       [tokens, rotary_dim] table holding [cos(theta) | sin(theta)] (theta of width
 *       rotary_dim/2), half-split pairs (d, d + rotary_dim/2) or interleaved pairs (2i, 2i+1).
 *   [3D form] FlashInfer "flashinfer.norm.fused_qk_rmsnorm_rope", description and parameters:
 *       across-heads RMSNorm of Q and K, RoPE computed from a frame/height/width decomposition of
 *       the token index (optionally YaRN-scaled), V copied out of the packed QKV input, and
 *       optional FP8 E4M3 outputs.
 *
 * Conventions shared by every entry point:
 *   - All functions return a qkrope_status, and on any status other than QKROPE_OK
 *     qkrope_last_error() returns a message for the calling thread. QKROPE_ERR_INVALID and
 *     QKROPE_ERR_UNSUPPORTED are found before anything is launched. A call whose grid would
 *     exceed one dispatch (2^32 - 1 lanes, e.g. past 2^26 tokens with 64-lane workgroups) runs
 *     as several launches over consecutive token ranges, in order on `stream`. A
 *     QKROPE_ERR_DEVICE from one of those launches leaves the earlier ranges enqueued and the
 *     later ones not.
 *   - Tensor pointers are DEVICE pointers, owned by the caller. The library never allocates,
 *     frees, or synchronises on them; it only enqueues work on `stream` (a hipStream_t; NULL is
 *     the default stream) and returns. A kernel fault therefore surfaces at the caller's next
 *     synchronisation with that stream.
 *   - Activations are bf16 (qkrope_run_table_ex also takes IEEE binary16), passed as raw 16-bit
 *     patterns. Every 16-bit tensor pointer must be 16-byte aligned and every token stride a
 *     multiple of 8 elements (one 16-byte chunk), else QKROPE_ERR_UNSUPPORTED.
 *   - Arithmetic is fp32 on the GPU; each output element is rounded once (to the 16-bit format
 *     round-to-nearest-even, or OCP E4M3 round-to-nearest-even with saturation to +-448).
 *   - A handle is immutable after qkrope_create, so calls on different streams may run
 *     concurrently from several host threads.
 */
#ifndef QKROPE_H
#define QKROPE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qkrope_status {
    QKROPE_OK = 0,
    QKROPE_ERR_INVALID = 1,      /* arguments break the pages' contract (shape, divisibility...) */
    QKROPE_ERR_UNSUPPORTED = 2,  /* valid per the pages but outside this library's kernels
                                    (alignment, head_dim or head-count limits) */
    QKROPE_ERR_DEVICE = 3,       /* HIP runtime error: device query, wrong architecture, launch */
    QKROPE_ERR_ALLOC = 4         /* host memory for the handle could not be allocated */
} qkrope_status;

/* Element formats. bf16 and IEEE binary16 (F16) are 16-bit activations; F32 appears only in
 * RoPE tables; E4M3 is the OCP FP8 output format (one byte per element). */
enum { QKROPE_DTYPE_BF16 = 0, QKROPE_DTYPE_F32 = 1, QKROPE_DTYPE_F16 = 2, QKROPE_DTYPE_E4M3 = 3 };

/* rope_table element types for qkrope_run_table: the table form's page allows the activation
 * dtype (bf16) or float32. */
enum { QKROPE_TABLE_BF16 = QKROPE_DTYPE_BF16, QKROPE_TABLE_F32 = QKROPE_DTYPE_F32 };

/* Norm modes for qkrope_run_table. PER_HEAD is the table form's contract (weights [head_dim],
 * one RMS per head). ACROSS_HEADS (weights [heads*head_dim], one RMS over the token's whole Q or
 * K row, as in the 3D form) and NONE (RoPE only) extend the table form so it covers every norm
 * the 3D form has. */
enum { QKROPE_NORM_NONE = 0, QKROPE_NORM_PER_HEAD = 1, QKROPE_NORM_ACROSS_HEADS = 2 };

typedef struct qkrope_ctx *qkrope_handle;

/* Create a handle bound to HIP device `device_ordinal` (made current for the query). Fails with
 * QKROPE_ERR_DEVICE if the device is not a gfx950 part. *out receives the handle. */
int qkrope_create(int device_ordinal, qkrope_handle *out);

/* Release a handle. NULL is accepted and ignored. No device work is pending on a handle (it holds
 * only a snapshot of device properties), so this never blocks. */
int qkrope_destroy(qkrope_handle h);

/* Static text for a status code. */
const char *qkrope_status_str(int status);

/* Detail of the last error on the calling thread ("" after a successful call). */
const char *qkrope_last_error(void);

/*
 * Fused-vs-eager token threshold (vLLM-Omni "vllm_omni.diffusion.layers.fused_qk_norm_rope",
 * fused_qk_norm_rope_min_tokens): below some number of tokens per call a fused call is bound by
 * host dispatch and a consumer may keep its eager chain. The caller passes the threshold it
 * measured (`default_tokens`, >= 0); a deployment overrides it for every caller through the
 * environment variable QKROPE_FUSED_MIN_TOKENS, read at every call (nothing is cached):
 *   unset, empty or only blanks  -> default_tokens;
 *   a non-negative decimal integer (surrounding blanks allowed) -> that value, 0 = always fuse;
 *   anything else -> QKROPE_ERR_INVALID (and *out is left unchanged).
 * Host-only; touches no device.
 */
int qkrope_min_tokens(int64_t default_tokens, int64_t *out);

/*
 * Table form (vLLM-Omni fused_qk_norm_rope).
 *
 *   q          [num_tokens, num_heads_q, head_dim] bf16; token t starts at q + t*q_token_stride
 *              (elements); heads and dims are contiguous inside a token.
 *   k          [num_tokens, num_heads_k, head_dim] bf16, token stride k_token_stride.
 *   q_weight,  norm weights, bf16: [head_dim] for PER_HEAD, [num_heads*head_dim] for
 *   k_weight   ACROSS_HEADS, ignored (may be NULL) for NONE.
 *   rope_table [num_tokens, rotary_dim], token stride table_token_stride (elements), dtype
 *              table_dtype. Row t holds cos(theta_t,i) for i < rotary_dim/2, then sin(theta_t,i).
 *              Row t rotates token t.
 *   eps        RMSNorm epsilon: n = x * (mean(x^2) + eps)^(-1/2) * w.
 *   rotary_dim even, 0 <= rotary_dim <= head_dim; dims >= rotary_dim are normalised, not
 *              rotated (rotary_dim 0: RoPE is skipped and rope_table may be NULL).
 *   interleaved 0: half-split pairs (i, i + rotary_dim/2); 1: adjacent pairs (2i, 2i + 1).
 *   q_out,     outputs with the inputs' shapes, bf16, token strides *_out_token_stride.
 *   k_out      q_out == q (with equal strides) works in place, likewise k_out == k; any other
 *              overlap between an output and an input is QKROPE_ERR_INVALID.
 *
 * Limits (else QKROPE_ERR_UNSUPPORTED): head_dim a multiple of 8 and <= 256; num_tokens < 2^31;
 * q, k and output token strides multiples of 8 elements and < 2^28; heads * L <= 4096 for each
 * of Q and K, L being head_dim / 8 rounded up to a power of two (e.g. 256 heads of 128). Any
 * even rotary_dim works with either pairing (half-split partners that straddle 16-byte
 * chunks, i.e. rotary_dim % 16 != 0, are exchanged through LDS, a slower path).
 * num_tokens == 0 (or zero heads) is a valid no-op.
 */
int qkrope_run_table(qkrope_handle h,
                     const void *q, const void *k, const void *q_weight, const void *k_weight,
                     const void *rope_table, int table_dtype, double eps,
                     int64_t num_tokens, int num_heads_q, int num_heads_k, int head_dim,
                     int rotary_dim, int interleaved, int norm_mode,
                     int64_t q_token_stride, int64_t k_token_stride, int64_t table_token_stride,
                     void *q_out, void *k_out,
                     int64_t q_out_token_stride, int64_t k_out_token_stride,
                     void *stream);

/*
 * Table form, extended contract. Everything qkrope_run_table does, plus:
 *   - separate cosine and sine tables, each [num_tokens, rotary_dim/2] with its own token stride
 *     (the layout of the rope_cos / rope_sin tables of vLLM-Omni's SANA-WM camera prologue,
 *     "vllm_omni.diffusion.models.sana_wm.ucpe", cam_prep_func parameters); row t of cos_table
 *     holds cos(theta_t,i), row t of sin_table sin(theta_t,i), i < rotary_dim/2. A packed
 *     [cos | sin] table is cos_table = table, sin_table = table + rotary_dim/2 with equal strides.
 *   - act_dtype QKROPE_DTYPE_BF16 or QKROPE_DTYPE_F16: format of q, k and the norm weights (the
 *     table form's page ties the table dtype and outputs to "the activation dtype");
 *     table_dtype is QKROPE_DTYPE_F32 or equal to act_dtype.
 *   - out_dtype equal to act_dtype (each output rounded once, to nearest even), or
 *     QKROPE_DTYPE_E4M3: outputs are OCP E4M3 bytes of y * out_scale (round to nearest even,
 *     finite overflow and infinities saturating to +-448, a NaN giving the NaN code 0xFF),
 *     as the 3D form's output_fp8 does; then
 *     out_scale must be finite and > 0 (it is ignored otherwise), the output token strides count
 *     bytes, outputs must be 8-byte aligned, and no output may alias an input.
 * In-place use (q_out == q with equal strides) needs out_dtype == act_dtype. Other arguments,
 * limits and errors are those of qkrope_run_table.
 */
int qkrope_run_table_ex(qkrope_handle h,
                        const void *q, const void *k, const void *q_weight, const void *k_weight,
                        const void *cos_table, const void *sin_table, int table_dtype,
                        int act_dtype, int out_dtype, double out_scale, double eps,
                        int64_t num_tokens, int num_heads_q, int num_heads_k, int head_dim,
                        int rotary_dim, int interleaved, int norm_mode,
                        int64_t q_token_stride, int64_t k_token_stride,
                        int64_t cos_token_stride, int64_t sin_token_stride,
                        void *q_out, void *k_out,
                        int64_t q_out_token_stride, int64_t k_out_token_stride,
                        void *stream);

/*
 * 3D form (FlashInfer fused_qk_rmsnorm_rope).
 *
 *   qkv        [num_tokens, (num_heads_q + num_heads_k + num_heads_v) * head_dim] bf16,
 *              contiguous; each row holds the token's Q heads, then K heads, then V heads.
 *              num_tokens = batch * seq_len must be a multiple of seq_len = ppf*pph*ppw; token t
 *              sits at grid position s = t mod seq_len, frame-major:
 *              f = s / (pph*ppw), h = (s / ppw) mod pph, w = s mod ppw.
 *   q_weight,  RMSNorm weights [num_heads_q*head_dim] and [num_heads_k*head_dim], bf16, used
 *   k_weight   when is_qk_norm != 0 (one RMS over each token's whole Q, resp. K, row);
 *              ignored (may be NULL) otherwise.
 *   num_*_channels  even, summing to head_dim. The head_dim/2 rotation pairs take their
 *              frequency from the concatenation [frame | height | width]: pair j of an axis with
 *              C channels has omega_j = base^(-2j/C) and angle pos_axis * omega'_j.
 *   head_dim   64, 128 or 256.
 *   interleave 1: pairs (2k, 2k+1); 0: NeoX pairs (k, k + head_dim/2).
 *   factor, low, high, attention_factor  YaRN. factor == 1 disables it and then
 *              attention_factor must be 1. Otherwise high > low and, per axis pair index j,
 *              rho = clamp((j - low)/(high - low), 0, 1),
 *              omega'_j = (omega_j/factor)*rho + omega_j*(1 - rho); cos and sin are multiplied by
 *              attention_factor.
 *   output_fp8 0: q_out/k_out/v_out are bf16; V is a bit copy.
 *              1: they are OCP E4M3 bytes: Q/K = e4m3(y * output_quant_scale),
 *              V = e4m3(v * v_quant_scale), round to nearest even, finite overflow and
 *              infinities saturating to +-448, a NaN giving the NaN code 0xFF (the hardware
 *              conversion's, whatever the NaN's sign); scales must be finite and > 0.
 *   q_out, k_out, v_out  [num_tokens, num_heads_x, head_dim], contiguous, and must not overlap
 *              qkv or each other.
 *
 * Limits (else QKROPE_ERR_UNSUPPORTED): num_tokens < 2^31; seq_len = ppf*pph*ppw < 2^31; one
 * workgroup per token covers at most 2048 16-byte chunks (heads * head_dim / 8) in each of Q, K
 * and V (e.g. 128 heads of 128 in each), or 4096 in all three together. num_tokens == 0 is a
 * valid no-op.
 */
int qkrope_run_3d(qkrope_handle h,
                  const void *qkv, const void *q_weight, const void *k_weight, int64_t num_tokens,
                  int ppf, int pph, int ppw,
                  int num_frame_channels, int num_height_channels, int num_width_channels,
                  int num_heads_q, int num_heads_k, int num_heads_v, int head_dim,
                  double eps, double base, int interleave, double factor, double low,
                  double high, double attention_factor, int is_qk_norm, int output_fp8,
                  double output_quant_scale, double v_quant_scale,
                  void *q_out, void *k_out, void *v_out, void *stream);

/*
 * Sharded 3D form: the pieces one rank of a sequence- or head-sharded run needs.
 *
 * The FlashInfer page defines the across-heads norm over a token's whole Q (K) row; vLLM-Omni's
 * SANA-WM page ("vllm_omni.diffusion.models.sana_wm.ucpe", cam_prep_func) notes that under
 * tensor parallelism the norm must still span every channel, not only a shard's. A rank whose
 * qkv holds only some heads of each token therefore (1) computes per-token partial sums of
 * squares of its Q and K heads with qkrope_sumsq_3d, (2) sums them over the ranks of its
 * head group (an all-reduce, the caller's), and (3) passes the totals to qkrope_run_3d_sharded.
 * A rank that holds a contiguous slice of tokens passes the slice's first global token index
 * as token_offset, so that every token keeps its (frame, height, width) position.
 */

/* sumsq[2t] = sum of x^2 over token t's num_heads_q*head_dim Q values in qkv,
 * sumsq[2t+1] = the same over its K values; fp32, accumulated in fp32. qkv has the layout of
 * qkrope_run_3d (num_heads_v heads of V after K; they are not read). sumsq is a device array
 * of 2*num_tokens floats, 8-byte aligned, not overlapping qkv. head_dim must be a multiple of
 * 8; (num_heads_q + num_heads_k) * head_dim / 8 <= 8192. num_tokens == 0 is a no-op. */
int qkrope_sumsq_3d(qkrope_handle h, const void *qkv, int64_t num_tokens, int num_heads_q,
                    int num_heads_k, int num_heads_v, int head_dim, float *sumsq, void *stream);

/* qkrope_run_3d on a shard:
 *   token_offset  global index of qkv's first token: token t sits at grid position
 *                 (token_offset + t) mod (ppf*pph*ppw). num_tokens need not be a multiple of
 *                 ppf*pph*ppw; token_offset >= 0 and token_offset + num_tokens < 2^31
 *                 (ppf*pph*ppw < 2^31 as for qkrope_run_3d).
 *   sumsq         NULL: the norm spans the shard's own heads (as qkrope_run_3d).
 *                 Otherwise (with is_qk_norm) a device array [num_tokens, 2] of fp32 sums of
 *                 squares of each token's Q and K rows over ALL heads of the unsharded problem
 *                 (the reduced output of qkrope_sumsq_3d), 8-byte aligned; the norm is then
 *                 x * (sumsq / norm_elems + eps)^(-1/2) * w, where norm_elems_q/k are the
 *                 element counts the sums cover (num_heads_q_total * head_dim, ...) and must be
 *                 >= the shard's own; q_weight/k_weight are the shard's slices [num_heads * D].
 *                 norm_elems_* are ignored when sumsq is NULL.
 * Every other argument is that of qkrope_run_3d. */
int qkrope_run_3d_sharded(qkrope_handle h,
                          const void *qkv, const void *q_weight, const void *k_weight,
                          int64_t num_tokens, int64_t token_offset, const float *sumsq,
                          int64_t norm_elems_q, int64_t norm_elems_k,
                          int ppf, int pph, int ppw,
                          int num_frame_channels, int num_height_channels, int num_width_channels,
                          int num_heads_q, int num_heads_k, int num_heads_v, int head_dim,
                          double eps, double base, int interleave, double factor, double low,
                          double high, double attention_factor, int is_qk_norm, int output_fp8,
                          double output_quant_scale, double v_quant_scale,
                          void *q_out, void *k_out, void *v_out, void *stream);

/*
 * Camera prologue of the SANA-WM UCPE branch: vLLM-Omni "vllm_omni.diffusion.models.sana_wm.ucpe",
 * cam_prep_func (parameters and returns). The page lists the steps (ReLU, the K scale, the
 * per-token 4x4 ray projection, interleaved RoPE from separate cos and sin tables) and the
 * shapes, but not how they compose; this library takes the reading
 *     q_trans = RoPE(P_q . ReLU(q))
 *     k_trans = RoPE(P_kv . (k_scale * ReLU(k)))
 *     v_trans = RoPE(P_kv . v)
 *     inflation_sq = |P_kv . k'|^2 / |k'|^2 with k' = k_scale * ReLU(k)   (1 where k' = 0)
 * per batch b, token n and head h, where P . x applies the token's 4x4 matrix to each group of
 * four consecutive channels, y[4g+i] = sum_j P[i][j] * x[4g+j], and RoPE rotates the pairs
 * (2i, 2i+1) by +theta: (a, b) -> (a cos - b sin, b cos + a sin) with cos = rope_cos[n][i],
 * sin = rope_sin[n][i]. ReLU(x) = x for x > 0 and for a NaN of either sign (the page does not
 * say what a NaN becomes; PyTorch's ReLU, whose native equivalent the page presents, keeps it),
 * +0 otherwise; a NaN in a key head makes its inflation_sq NaN. The RMSNorm of q and k is the
 * caller's.
 *
 *   q, k, v        device, [batch, num_tokens, num_heads, head_dim] activations (act_dtype bf16
 *                  or binary16); token (b, n) starts at (b*num_tokens + n) * x_stride elements;
 *                  16-byte aligned; strides multiples of 8, >= num_heads*head_dim, < 2^24.
 *                  The three may alias (all are read-only).
 *   proj_q, proj_kv  device float32 [batch, num_tokens, 4, 4], row-major per token, 16-byte
 *                  aligned.
 *   rope_cos, rope_sin  device float32 [num_tokens, head_dim/2], 16-byte aligned.
 *   k_scale        multiplies K (the page's head_dim^-1/2 * spatial_tokens^-1/2).
 *   q_out, k_out, v_out  device, [batch, num_heads, head_dim, num_tokens] in act_dtype, 2-byte
 *                  aligned; row (b, h, d) of each starts at ((b*num_heads + h)*head_dim + d) *
 *                  out_row_stride elements and holds the num_tokens values; elements between
 *                  num_tokens and out_row_stride are not written.
 *   out_row_stride elements between consecutive output rows, >= num_tokens and < 2^31
 *                  (num_tokens: contiguous outputs). With 16-byte aligned outputs and a stride
 *                  that is a multiple of 8, whole 64-token tiles take 16-byte stores; a stride
 *                  that is a multiple of 64 (with 128-byte aligned outputs) starts every row on
 *                  a 128-byte line, which these stores write fastest.
 *   inflation_sq   device float32 [batch, num_heads, num_tokens], contiguous, or NULL to skip.
 * No output may overlap an input or another output (their whole row spans, padding included).
 * head_dim must be a multiple of 4 and out_row_stride >= num_tokens (QKROPE_ERR_INVALID
 * otherwise); this library handles multiples of 8 up to 256,
 * batch * num_tokens < 2^31, and grids of at most 2^32 - 1 lanes (one launch; first exceeded
 * with a single head of 64 past 2^29 (b, n) tokens) (QKROPE_ERR_UNSUPPORTED). An empty problem
 * (batch, num_tokens or num_heads 0) is a no-op.
 */
int qkrope_cam_prep(qkrope_handle h, const void *q, const void *k, const void *v, int act_dtype,
                    const float *proj_q, const float *proj_kv, const float *rope_cos,
                    const float *rope_sin, float k_scale, int64_t batch, int64_t num_tokens,
                    int num_heads, int head_dim, int64_t q_stride, int64_t k_stride,
                    int64_t v_stride, void *q_out, void *k_out, void *v_out,
                    int64_t out_row_stride, float *inflation_sq, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QKROPE_H */
