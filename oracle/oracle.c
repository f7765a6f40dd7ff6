/*
 * oracle.c -- plain, slow, fp64 CPU oracle for the fused QK-RMSNorm + RoPE (+ V) prologue.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and the benchmark's
 * CPU-baseline leg load this library. It shares no code, header, table or helper with the HIP
 * path, and the HIP path never calls it.
 *
 * What it follows (the pages, cited by title and section):
 *   [table form] vLLM-Omni API docs, "vllm_omni.diffusion.layers.fused_qk_norm_rope",
 *       module contract: q/k are [tokens, heads, head_dim]; the norm weights are [head_dim];
 *       rope_table is [tokens, rotary_dim] holding [cos(theta) | sin(theta)], theta of width
 *       rotary_dim/2, in the activation dtype or float32; interleaved=False rotates the pairs
 *       (d, d + rotary_dim/2), interleaved=True the adjacent pairs (2i, 2i+1) by theta_i.
 *       The fused path materialises no normalised or rotated intermediates.
 *   [split tables] vLLM-Omni API docs, "vllm_omni.diffusion.models.sana_wm.ucpe", cam_prep_func
 *       parameters: separate (N, D/2) cosine and sine tables for interleaved pairs.
 *   [3D form] FlashInfer API docs, "flashinfer.norm.fused_qk_rmsnorm_rope", description and
 *       parameter list: across-heads RMSNorm of Q and K (weights [heads*head_dim]); RoPE with a
 *       frame/height/width decomposition (seq_len = ppf*pph*ppw, channel counts per axis that
 *       sum to head_dim, frequency base); interleave=True for adjacent pairs, False for NeoX;
 *       YaRN factor/low/high and an attention factor applied to cos and sin; is_qk_norm=False
 *       skips the norm; V is copied out of packed QKV; optional FP8 E4M3 outputs with one scale
 *       for Q and K and one for V.
 *
 * Where the pages leave a step open, the reading taken is stated next to the code:
 *   - RMSNorm: n = x * (mean(x^2) + eps)^(-1/2) * w, eps inside the root, w multiplied directly.
 *   - rotation by +theta: a' = a*cos - b*sin, b' = b*cos + a*sin.
 *   - dims at or beyond rotary_dim are normalised but not rotated.
 *   - 3D positions are frame-major (width fastest); token t of a flattened batch is position
 *     t mod seq_len. The frequency vector of length head_dim/2 is the concatenation of the frame,
 *     height and width blocks; block pair j has omega = base^(-2j/C_axis). NeoX pairs (k, k+D/2)
 *     across that whole vector.
 *   - YaRN: per axis, ramp rho = clamp((j - low)/(high - low), 0, 1) over the block pair index,
 *     omega' = (omega/factor)*rho + omega*(1 - rho) (the published YaRN blend of interpolated and
 *     original frequencies); cos and sin are then multiplied by attention_factor.
 *   - FP8: OCP E4M3 (bias 7, max 448, no infinities, NaN = S.1111.111), round to nearest even,
 *     value multiplied by its scale, finite overflow saturates to +-448.
 *   - "Activation dtype" covers bf16 and IEEE binary16; weights share the activation dtype.
 *   - A head-sharded across-heads norm uses the sums of squares of the whole row (every shard's
 *     heads), i.e. it equals the unsharded norm; oracle_sumsq_3d gives those per-token sums.
 *   [camera prologue] vLLM-Omni API docs, "vllm_omni.diffusion.models.sana_wm.ucpe",
 *       cam_prep_func: Q, K (already normalised) and raw V are (B, N, H, D); proj_q and proj_kv
 *       are per-token (B, N, 4, 4) ray projection matrices; rope_cos / rope_sin are (N, D/2)
 *       interleaved-pair tables; k_scale multiplies K; the steps are ReLU, the K scale, the ray
 *       projection and RoPE; outputs are (B, H, D, N) plus inflation_sq (B, H, N). The page
 *       names these but leaves open how they compose; the readings taken here:
 *   - Q: ReLU, projection by proj_q, RoPE. K: ReLU, times k_scale, projection by proj_kv, RoPE.
 *     V: projection by proj_kv, RoPE (the K/V matrices are one transform shared by K and V).
 *     ReLU(x) = x for x > 0, 0 for every other number (negatives and both zeros give +0), and
 *     a NaN of either sign stays NaN. The page does not say what a NaN becomes; it presents
 *     cam_prep_func as the native equivalent of a PyTorch module, and PyTorch's ReLU passes
 *     every NaN through, so this reading does too.
 *   - A 4x4 matrix P acts on a head vector as D/4 independent groups of four consecutive
 *     channels: y[4g + i] = sum_j P[i][j] * x[4g + j], P stored row-major.
 *   - RoPE rotates the adjacent pairs (2i, 2i+1) of the projected vector by the angle whose
 *     cosine and sine are row n, column i of the tables (rotation by +theta as above).
 *   - inflation_sq(b, h, n) = |P_kv applied to k'|^2 / |k'|^2 for the key head vector
 *     k' = k_scale * ReLU(k) that enters the projection (how much the projection grows its
 *     squared norm), and 1 where |k'| = 0; a NaN in k' makes it NaN (the quotient's own
 *     value).
 *
 * Everything is computed in double from the exact decoded inputs and rounded once at the output.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_OK = 0, ORACLE_BAD_ARG = 1, ORACLE_NO_MEMORY = 2 };
enum { ORACLE_NORM_NONE = 0, ORACLE_NORM_PER_HEAD = 1, ORACLE_NORM_ACROSS_HEADS = 2 };
/* Table dtypes: the pages allow the activation dtype (bf16) or float32. F64 is a test-only
 * extension that lets the table form be compared exactly with the 3D form. */
enum { ORACLE_TABLE_BF16 = 0, ORACLE_TABLE_F32 = 1, ORACLE_TABLE_F64 = 2, ORACLE_TABLE_F16 = 3 };
/* 16-bit activation formats. */
enum { ORACLE_ACT_BF16 = 0, ORACLE_ACT_F16 = 1 };

/* ---------------------------------------------------------------------------------------------
 * Number formats.
 * bf16 is the upper half of an IEEE-754 binary32; decoding is exact.
 * ------------------------------------------------------------------------------------------- */
double oracle_bf16_decode(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* IEEE-754 binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits; exponent 0 holds zero
 * and subnormals (fraction * 2^-24), exponent 31 infinities and NaNs. Decoding is exact. */
double oracle_f16_decode(uint16_t h)
{
    int s = h >> 15, E = (h >> 10) & 31, M = h & 1023;
    double v;
    if (E == 31) v = M ? NAN : INFINITY;
    else if (E == 0) v = ldexp((double)M, -24);
    else v = ldexp(1.0 + M / 1024.0, E - 15);
    return s ? -v : v;
}

double oracle_f32_decode(uint32_t u)
{
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round |a| (finite, > 0) to a binary grid with `prec` significant bits whose smallest normal
 * binade starts at 2^emin (below it the quantum stays 2^(emin - prec + 1)). Ties go to even:
 * rint() runs in the default round-to-nearest-even mode, and a/quantum is exact because the
 * quantum is a power of two. */
static double round_to_grid(double a, int prec, int emin)
{
    int e;
    frexp(a, &e);               /* a = m * 2^e, m in [0.5, 1): leading bit has weight 2^(e-1) */
    int lead = e - 1;
    if (lead < emin) lead = emin;
    double quantum = ldexp(1.0, lead - (prec - 1));
    return rint(a / quantum) * quantum;
}

/* bf16 round-to-nearest-even of an fp64 value (8 significant bits, exponent range of binary32).
 * Overflow rounds to infinity; NaN becomes a quiet NaN with its sign. */
uint16_t oracle_bf16_encode(double x)
{
    if (isnan(x)) return signbit(x) ? 0xFFC0 : 0x7FC0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a == 0.0) return sign;
    if (isinf(a)) return sign | 0x7F80;
    double r = round_to_grid(a, 8, -126);
    double max_finite = ldexp(255.0, 120);          /* (2 - 2^-7) * 2^127 */
    if (r > max_finite) return sign | 0x7F80;
    float f = (float)r;                             /* exact: r is on the bf16 grid */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (u >> 16));
}

/* binary16 round-to-nearest-even of an fp64 value (11 significant bits, smallest normal
 * 2^-14, largest finite 65504). Overflow rounds to infinity; NaN becomes a quiet NaN. */
uint16_t oracle_f16_encode(double x)
{
    if (isnan(x)) return signbit(x) ? 0xFE00 : 0x7E00;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a == 0.0) return sign;
    if (isinf(a)) return sign | 0x7C00;
    double r = round_to_grid(a, 11, -14);
    if (r > 65504.0) return sign | 0x7C00;
    if (r == 0.0) return sign;
    if (r < ldexp(1.0, -14))                        /* subnormal: fraction counts 2^-24 steps */
        return (uint16_t)(sign | (int)(r / ldexp(1.0, -24)));
    int e;
    frexp(r, &e);
    int lead = e - 1;                               /* r in [2^lead, 2^(lead+1)) */
    int mant = (int)((r / ldexp(1.0, lead) - 1.0) * 1024.0);
    return (uint16_t)(sign | ((lead + 15) << 10) | mant);
}

void oracle_encode_f16_array(const double *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_encode(x[i]);
}

/* OCP FP8 E4M3 ("e4m3fn"): 1 sign, 4 exponent (bias 7), 3 mantissa bits; normal binades
 * 2^-6 .. 2^8, subnormal quantum 2^-9, largest finite 448 = 1.75 * 2^8, no infinities, and
 * S.1111.111 is NaN. */
uint8_t oracle_e4m3_encode(double x)
{
    if (isnan(x)) return signbit(x) ? 0xFF : 0x7F;
    uint8_t sign = signbit(x) ? 0x80 : 0;
    double a = fabs(x);
    if (a > 448.0) a = 448.0;                       /* saturate (also maps +-inf to +-448) */
    if (a == 0.0) return sign;
    double r = round_to_grid(a, 4, -6);
    if (r == 0.0) return sign;
    if (r < ldexp(1.0, -6)) {                       /* subnormal: mantissa counts 2^-9 steps */
        return (uint8_t)(sign | (int)(r / ldexp(1.0, -9)));
    }
    int e;
    frexp(r, &e);
    int lead = e - 1;                               /* r in [2^lead, 2^(lead+1)) */
    int mant = (int)((r / ldexp(1.0, lead) - 1.0) * 8.0);
    return (uint8_t)(sign | ((lead + 7) << 3) | mant);
}

double oracle_e4m3_decode(uint8_t c)
{
    int s = c >> 7, E = (c >> 3) & 15, M = c & 7;
    double v;
    if (E == 15 && M == 7) return s ? -NAN : NAN;
    if (E == 0) v = ldexp((double)M, -9);
    else v = ldexp(1.0 + M / 8.0, E - 7);
    return s ? -v : v;
}

void oracle_encode_bf16_array(const double *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_encode(x[i]);
}

/* FP8 output of the 3D form: code = e4m3(value * scale). */
void oracle_quantize_e4m3_array(const double *x, int64_t n, double scale, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(x[i] * scale);
}

/* ---------------------------------------------------------------------------------------------
 * RMSNorm: the reciprocal root mean square of n values, (mean(x^2) + eps)^(-1/2).
 * ------------------------------------------------------------------------------------------- */
static double inv_rms(const double *x, int64_t n, double eps)
{
    double sum = 0.0;
    for (int64_t i = 0; i < n; ++i) sum += x[i] * x[i];
    return 1.0 / sqrt(sum / (double)n + eps);
}

static double act_decode(int act, uint16_t b)
{
    return act == ORACLE_ACT_F16 ? oracle_f16_decode(b) : oracle_bf16_decode(b);
}

/* Normalise one token's [H, D] block x in place. PER_HEAD: one scale per head, weight w[d].
 * ACROSS_HEADS: one scale for the whole H*D row, weight w[h*D + d]. NONE: unchanged. */
static void normalise_token(double *x, int H, int D, int norm_mode, const uint16_t *w, int act,
                            double eps)
{
    if (norm_mode == ORACLE_NORM_PER_HEAD) {
        for (int h = 0; h < H; ++h) {
            double r = inv_rms(x + (int64_t)h * D, D, eps);
            for (int d = 0; d < D; ++d)
                x[h * D + d] = x[h * D + d] * r * act_decode(act, w[d]);
        }
    } else if (norm_mode == ORACLE_NORM_ACROSS_HEADS) {
        double r = inv_rms(x, (int64_t)H * D, eps);
        for (int i = 0; i < H * D; ++i)
            x[i] = x[i] * r * act_decode(act, w[i]);
    }
}

/* ---------------------------------------------------------------------------------------------
 * Table form.
 * q: [T, Hq, D] 16-bit activations (bf16 or binary16) with token stride q_stride (elements);
 * k likewise; weights in the activation format. cos_table / sin_table: [T, R/2] each, with
 * their own token strides, dtype bf16, binary16, f32 (or f64 for tests); the pages' packed
 * [T, R] = [cos | sin] table is sin_table = cos_table + R/2. Outputs: fp64 [T, H, D], unrounded.
 * norm_mode PER_HEAD is the pages' contract ([head_dim] weights); NONE and ACROSS_HEADS
 * (weights [H*D]) are extensions used to relate the table form to the 3D form.
 * ------------------------------------------------------------------------------------------- */
static double table_value(const void *table, int dtype, int64_t idx)
{
    if (dtype == ORACLE_TABLE_F64) return ((const double *)table)[idx];
    if (dtype == ORACLE_TABLE_F32) return oracle_f32_decode(((const uint32_t *)table)[idx]);
    if (dtype == ORACLE_TABLE_F16) return oracle_f16_decode(((const uint16_t *)table)[idx]);
    return oracle_bf16_decode(((const uint16_t *)table)[idx]);
}

static void table_token(const uint16_t *src, int act, int H, int D, int R, int interleaved,
                        int norm_mode, const uint16_t *w, double eps,
                        const void *cos_table, const void *sin_table, int dtype,
                        int64_t cos_row, int64_t sin_row, double *out, double *n)
{
    for (int i = 0; i < H * D; ++i) n[i] = act_decode(act, src[i]);
    normalise_token(n, H, D, norm_mode, w, act, eps);
    for (int h = 0; h < H; ++h) {
        const double *nh = n + (int64_t)h * D;
        double *oh = out + (int64_t)h * D;
        for (int d = 0; d < D; ++d) oh[d] = nh[d];            /* dims >= R pass through */
        for (int i = 0; i < R / 2; ++i) {
            double c = table_value(cos_table, dtype, cos_row + i);
            double s = table_value(sin_table, dtype, sin_row + i);
            int a = interleaved ? 2 * i : i;
            int b = interleaved ? 2 * i + 1 : i + R / 2;
            oh[a] = nh[a] * c - nh[b] * s;
            oh[b] = nh[b] * c + nh[a] * s;
        }
    }
}

int oracle_run_table_split(const uint16_t *q, const uint16_t *k,
                           const uint16_t *q_weight, const uint16_t *k_weight, int act_dtype,
                           const void *cos_table, const void *sin_table, int table_dtype,
                           double eps, int64_t num_tokens, int num_heads_q, int num_heads_k,
                           int head_dim, int rotary_dim, int interleaved, int norm_mode,
                           int64_t q_stride, int64_t k_stride, int64_t cos_stride,
                           int64_t sin_stride, double *q_out, double *k_out)
{
    if (num_tokens < 0 || num_heads_q < 0 || num_heads_k < 0 || head_dim <= 0) return ORACLE_BAD_ARG;
    if (rotary_dim < 0 || rotary_dim > head_dim || rotary_dim % 2) return ORACLE_BAD_ARG;
    if (norm_mode < 0 || norm_mode > 2) return ORACLE_BAD_ARG;
    if (act_dtype != ORACLE_ACT_BF16 && act_dtype != ORACLE_ACT_F16) return ORACLE_BAD_ARG;
    if (table_dtype < ORACLE_TABLE_BF16 || table_dtype > ORACLE_TABLE_F16) return ORACLE_BAD_ARG;
    int D = head_dim, R = rotary_dim;
    int Hmax = num_heads_q > num_heads_k ? num_heads_q : num_heads_k;
    int64_t T = num_tokens;
    int failed = 0;
#pragma omp parallel
    {
        double *scratch = (double *)malloc(sizeof(double) * ((size_t)Hmax * D + 1));
        if (!scratch) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            if (!scratch) continue;
            table_token(q + t * q_stride, act_dtype, num_heads_q, D, R, interleaved, norm_mode,
                        q_weight, eps, cos_table, sin_table, table_dtype, t * cos_stride,
                        t * sin_stride, q_out + t * num_heads_q * D, scratch);
            table_token(k + t * k_stride, act_dtype, num_heads_k, D, R, interleaved, norm_mode,
                        k_weight, eps, cos_table, sin_table, table_dtype, t * cos_stride,
                        t * sin_stride, k_out + t * num_heads_k * D, scratch);
        }
        free(scratch);
    }
    return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/* The pages' packed table: row t = [cos(theta_t,0..R/2-1) | sin(theta_t,0..R/2-1)], bf16
 * activations. */
int oracle_run_table(const uint16_t *q, const uint16_t *k,
                     const uint16_t *q_weight, const uint16_t *k_weight,
                     const void *rope_table, int table_dtype, double eps,
                     int64_t num_tokens, int num_heads_q, int num_heads_k, int head_dim,
                     int rotary_dim, int interleaved, int norm_mode,
                     int64_t q_stride, int64_t k_stride, int64_t table_stride,
                     double *q_out, double *k_out)
{
    int esize = table_dtype == ORACLE_TABLE_F64 ? 8 : (table_dtype == ORACLE_TABLE_F32 ? 4 : 2);
    if (rotary_dim < 0 || rotary_dim % 2) return ORACLE_BAD_ARG;
    const void *sin_table = rope_table ? (const char *)rope_table + (size_t)(rotary_dim / 2) * esize
                                       : NULL;
    return oracle_run_table_split(q, k, q_weight, k_weight, ORACLE_ACT_BF16, rope_table,
                                  sin_table, table_dtype, eps, num_tokens, num_heads_q,
                                  num_heads_k, head_dim, rotary_dim, interleaved, norm_mode,
                                  q_stride, k_stride, table_stride, table_stride, q_out, k_out);
}

/* ---------------------------------------------------------------------------------------------
 * 3D form.
 * ------------------------------------------------------------------------------------------- */

/* Position of sequence index s on the (frame, height, width) grid, frame-major. */
static void grid_position(int64_t s, int pph, int ppw, int64_t pos[3])
{
    pos[0] = s / ((int64_t)pph * ppw);
    pos[1] = (s / ppw) % pph;
    pos[2] = s % ppw;
}

/* cos/sin (times attention_factor) of pair k of the head_dim/2-long frequency vector. */
static void pair_angle(int k, const int64_t pos[3], const int C[3], double base, double factor,
                       double low, double high, double attention_factor, double *c, double *s)
{
    int axis = 0, j = k;
    while (j >= C[axis] / 2) {          /* blocks: frame C[0]/2 pairs, height, then width */
        j -= C[axis] / 2;
        ++axis;
    }
    double omega = pow(base, -2.0 * j / (double)C[axis]);
    if (factor != 1.0) {
        double rho = (j - low) / (high - low);
        if (rho < 0.0) rho = 0.0;
        if (rho > 1.0) rho = 1.0;
        omega = (omega / factor) * rho + omega * (1.0 - rho);
    }
    double theta = (double)pos[axis] * omega;
    *c = cos(theta) * attention_factor;
    *s = sin(theta) * attention_factor;
}

static void rope3d_region(const uint16_t *src, int H, int D, int interleave, int norm,
                          const uint16_t *w, double eps, const double *cs_c, const double *cs_s,
                          double *out, double *n)
{
    for (int i = 0; i < H * D; ++i) n[i] = oracle_bf16_decode(src[i]);
    normalise_token(n, H, D, norm ? ORACLE_NORM_ACROSS_HEADS : ORACLE_NORM_NONE, w,
                    ORACLE_ACT_BF16, eps);
    for (int h = 0; h < H; ++h) {
        const double *nh = n + (int64_t)h * D;
        double *oh = out + (int64_t)h * D;
        for (int k = 0; k < D / 2; ++k) {
            int a = interleave ? 2 * k : k;
            int b = interleave ? 2 * k + 1 : k + D / 2;
            oh[a] = nh[a] * cs_c[k] - nh[b] * cs_s[k];
            oh[b] = nh[b] * cs_c[k] + nh[a] * cs_s[k];
        }
    }
}

/* qkv: rows of (Hq+Hk+Hv)*D bf16 for tokens token_offset .. token_offset+num_tokens-1 of a
 * flattened [B*S] sequence (the offset lets a caller check a slice of a long input). Outputs are
 * fp64 [num_tokens, H, D], unrounded; V is the decoded input. */
int oracle_run_3d(const uint16_t *qkv, const uint16_t *q_weight, const uint16_t *k_weight,
                  int64_t num_tokens, int64_t token_offset,
                  int ppf, int pph, int ppw,
                  int num_frame_channels, int num_height_channels, int num_width_channels,
                  int num_heads_q, int num_heads_k, int num_heads_v, int head_dim,
                  double eps, double base, int interleave, double factor, double low,
                  double high, double attention_factor, int is_qk_norm,
                  double *q_out, double *k_out, double *v_out)
{
    int C[3] = {num_frame_channels, num_height_channels, num_width_channels};
    int D = head_dim;
    if (ppf <= 0 || pph <= 0 || ppw <= 0 || D <= 0 || D % 2) return ORACLE_BAD_ARG;
    if (num_tokens < 0 || token_offset < 0) return ORACLE_BAD_ARG;
    for (int a = 0; a < 3; ++a)
        if (C[a] < 0 || C[a] % 2) return ORACLE_BAD_ARG;
    if (C[0] + C[1] + C[2] != D) return ORACLE_BAD_ARG;
    if (factor != 1.0 && !(high > low)) return ORACLE_BAD_ARG;
    if (factor == 1.0 && attention_factor != 1.0) return ORACLE_BAD_ARG;
    int Hq = num_heads_q, Hk = num_heads_k, Hv = num_heads_v;
    int64_t row = (int64_t)(Hq + Hk + Hv) * D;
    int64_t S = (int64_t)ppf * pph * ppw;
    int Hmax = Hq > Hk ? Hq : Hk;
    int failed = 0;
#pragma omp parallel
    {
        double *scratch = (double *)malloc(sizeof(double) * ((size_t)Hmax * D + (size_t)D + 2));
        if (!scratch) {
#pragma omp atomic write
            failed = 1;
        }
        double *cs_c = scratch ? scratch + (size_t)Hmax * D : NULL;
        double *cs_s = scratch ? cs_c + D / 2 + 1 : NULL;
#pragma omp for schedule(static)
        for (int64_t i = 0; i < num_tokens; ++i) {
            if (!scratch) continue;
            int64_t pos[3];
            grid_position((token_offset + i) % S, pph, ppw, pos);
            for (int k = 0; k < D / 2; ++k)
                pair_angle(k, pos, C, base, factor, low, high, attention_factor,
                           &cs_c[k], &cs_s[k]);
            const uint16_t *src = qkv + i * row;
            rope3d_region(src, Hq, D, interleave, is_qk_norm, q_weight, eps, cs_c, cs_s,
                          q_out + i * Hq * D, scratch);
            rope3d_region(src + (int64_t)Hq * D, Hk, D, interleave, is_qk_norm, k_weight, eps,
                          cs_c, cs_s, k_out + i * Hk * D, scratch);
            for (int64_t e = 0; e < (int64_t)Hv * D; ++e)
                v_out[i * Hv * D + e] = oracle_bf16_decode(src[(int64_t)(Hq + Hk) * D + e]);
        }
        free(scratch);
    }
    return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/* Per-token sums of squares of the Q and K rows of packed bf16 qkv (rows of (Hq+Hk+Hv)*D):
 * out[2t] = sum of x^2 over the token's Hq*D Q values, out[2t+1] over its Hk*D K values. These
 * are the sums the across-heads norm of the 3D form takes its mean of. */
int oracle_sumsq_3d(const uint16_t *qkv, int64_t num_tokens, int num_heads_q, int num_heads_k,
                    int num_heads_v, int head_dim, double *out)
{
    if (num_tokens < 0 || num_heads_q < 0 || num_heads_k < 0 || num_heads_v < 0 || head_dim <= 0)
        return ORACLE_BAD_ARG;
    int64_t nq = (int64_t)num_heads_q * head_dim, nk = (int64_t)num_heads_k * head_dim;
    int64_t row = (int64_t)(num_heads_q + num_heads_k + num_heads_v) * head_dim;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < num_tokens; ++t) {
        const uint16_t *x = qkv + t * row;
        double sq = 0.0, sk = 0.0;
        for (int64_t i = 0; i < nq; ++i) {
            double v = oracle_bf16_decode(x[i]);
            sq += v * v;
        }
        for (int64_t i = 0; i < nk; ++i) {
            double v = oracle_bf16_decode(x[nq + i]);
            sk += v * v;
        }
        out[2 * t] = sq;
        out[2 * t + 1] = sk;
    }
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------------------------------
 * Camera prologue (UCPE page, cam_prep_func). q, k, v: [B, N, H, D] 16-bit activations with
 * token strides q_stride, k_stride, v_stride (elements; batch stride N * token stride).
 * proj_q, proj_kv: [B, N, 4, 4] float32, row-major per token. rope_cos, rope_sin: [N, D/2]
 * float32. Outputs, fp64 unrounded: q_out, k_out, v_out [B, H, D, N]; inflation_sq [B, H, N].
 * ------------------------------------------------------------------------------------------- */

/* p = P applied to each group of four channels of a (D values). */
static void project_groups(const float *P, const double *a, int D, double *p)
{
    for (int g = 0; g < D / 4; ++g)
        for (int i = 0; i < 4; ++i) {
            double acc = 0.0;
            for (int j = 0; j < 4; ++j)
                acc += (double)P[4 * i + j] * a[4 * g + j];
            p[4 * g + i] = acc;
        }
}

/* One head vector through the camera transform: ReLU if relu, times scale, projection, RoPE.
 * Writes y[0..D) and returns |p|^2 / |a|^2 (1 when |a| = 0), a and p as in the header. */
static double cam_head(const uint16_t *x, int act, int relu, double scale, const float *P,
                       const float *cos_row, const float *sin_row, int D, double *a, double *p,
                       double *y)
{
    double na = 0.0, np_ = 0.0;
    for (int d = 0; d < D; ++d) {
        double v = act_decode(act, x[d]);
        if (relu) v = (v > 0.0 || isnan(v)) ? v : 0.0;
        a[d] = scale * v;
        na += a[d] * a[d];
    }
    project_groups(P, a, D, p);
    for (int d = 0; d < D; ++d) np_ += p[d] * p[d];
    for (int i = 0; i < D / 2; ++i) {
        double c = (double)cos_row[i], s = (double)sin_row[i];
        y[2 * i] = p[2 * i] * c - p[2 * i + 1] * s;
        y[2 * i + 1] = p[2 * i + 1] * c + p[2 * i] * s;
    }
    return na == 0.0 ? 1.0 : np_ / na;
}

int oracle_cam_prep(const uint16_t *q, const uint16_t *k, const uint16_t *v, int act_dtype,
                    const float *proj_q, const float *proj_kv, const float *rope_cos,
                    const float *rope_sin, double k_scale, int64_t batch, int64_t num_tokens,
                    int num_heads, int head_dim, int64_t q_stride, int64_t k_stride,
                    int64_t v_stride, double *q_out, double *k_out, double *v_out,
                    double *inflation_sq)
{
    if (batch < 0 || num_tokens < 0 || num_heads < 0 || head_dim <= 0 || head_dim % 4)
        return ORACLE_BAD_ARG;
    if (act_dtype != ORACLE_ACT_BF16 && act_dtype != ORACLE_ACT_F16) return ORACLE_BAD_ARG;
    const int D = head_dim, H = num_heads;
    const int64_t N = num_tokens, BN = batch * num_tokens;
    int failed = 0;
#pragma omp parallel
    {
        double *scratch = (double *)malloc(sizeof(double) * 3 * (size_t)D);
        if (!scratch) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(static)
        for (int64_t bn = 0; bn < BN; ++bn) {
            if (!scratch) continue;
            const int64_t b = bn / N, n = bn % N;
            double *a = scratch, *p = scratch + D, *y = scratch + 2 * D;
            const float *cr = rope_cos + n * (D / 2), *sr = rope_sin + n * (D / 2);
            for (int h = 0; h < H; ++h) {
                const int64_t o = (b * H + h) * (int64_t)D * N + n;  /* out[b][h][0][n] */
                cam_head(q + bn * q_stride + (int64_t)h * D, act_dtype, 1, 1.0, proj_q + bn * 16,
                         cr, sr, D, a, p, y);
                for (int d = 0; d < D; ++d) q_out[o + (int64_t)d * N] = y[d];
                double infl = cam_head(k + bn * k_stride + (int64_t)h * D, act_dtype, 1, k_scale,
                                       proj_kv + bn * 16, cr, sr, D, a, p, y);
                for (int d = 0; d < D; ++d) k_out[o + (int64_t)d * N] = y[d];
                inflation_sq[(b * H + h) * N + n] = infl;
                cam_head(v + bn * v_stride + (int64_t)h * D, act_dtype, 0, 1.0, proj_kv + bn * 16,
                         cr, sr, D, a, p, y);
                for (int d = 0; d < D; ++d) v_out[o + (int64_t)d * N] = y[d];
            }
        }
        free(scratch);
    }
    return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/* Threads an OpenMP parallel region of this library will use. */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
