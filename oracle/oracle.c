/*
 * oracle.c -- plain, slow CPU reference for the FP8 (E4M3FN) per-row KV cache
 * and the GQA attention that reads it.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or load
 * this file: only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header, table or constant generator
 * with the HIP library; the only thing both sides share is the seeded input
 * generator, which holds none of this arithmetic.
 *
 * Sources (the pages are cited by title and section):
 *   [853]  FreeToken PR #853 "opt-in FP8 KV cache": "What changes" (each
 *          physical K/V row stores E4M3 code bytes plus its own FP32 scale;
 *          prefill rebuilds historical FP8 rows once per layer into one shared
 *          BF16 workspace while the current chunk stays BF16), "Validation"
 *          (pool byte accounting), "Follow-up model/workload search" (each new
 *          K/V row is quantized on write, per-row scales are loaded during
 *          attention).
 *   [897]  FreeToken PR #897 "perf(attention): add packed fp8 kv reads on
 *          gfx1201": description (E4M3FN codes, per-token/head scales, GQA 4/8,
 *          D=128 decode) and "Regression and CUDA isolation" (every finite
 *          E4M3FN value, signed zero included, must survive decode).
 *   [280]  FreeToken issue #280 "Feature Request: opt-in FP8 KV-cache support
 *          for long-context MoE inference": "Proof of concept" (E4M3 values
 *          with independent dynamic FP32 scales, dequantized inside attention)
 *          and "Current proof-of-concept limitations" (dynamic per-token /
 *          per-KV-head scales).
 *   [OFP8] OCP 8-bit Floating Point Specification (OFP8), E4M3 encoding: 1 sign
 *          bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
 *          encodes subnormals m * 2^-9; S.1111.111 is NaN; there is no infinity;
 *          the largest finite magnitude is 1.75 * 2^8 = 448.
 *
 * Readings the pages leave open (each is listed with its reason in the design
 * notes):
 *   - scale s = fl32(amax / 448) per (token, KV head), K and V separately; the
 *     division is a true IEEE fp32 division, not a reciprocal multiply.
 *   - every element is divided by s in fp32 (correctly rounded), then rounded
 *     to E4M3FN with round-to-nearest-even and saturation to +-448.
 *   - a row whose amax is 0 gets s = 0 and codes +0 / -0 (the input's sign).
 *   - query head h reads KV head floor(h / (Hq/Hkv)).
 *   - dequantized values decode(c) * s are formed exactly in fp64; attention is
 *     the plain softmax(q . K^T * sm_scale) . V in fp64.
 *   - the prefill workspace holds bf16_rne(fl32(decode(c) * s)).
 *   - chunk query i sees every prefix row and chunk rows 0..i.
 *   - head dim D is 128 or 256 ([897] "Regression and CUDA isolation": the
 *     comparison matrix covers D128 and D256).
 *   - a decode request may carry n_qrows query rows (up to 8: [897]
 *     description, the multi-row decode of #900; 1/3/8 query rows in
 *     "Regression and CUDA isolation"): they are its last n_qrows positions,
 *     each causal over the request's rows.
 *   - a sliding window of W keys ([897] "Regression and CUDA isolation": the
 *     integration cases include an odd sliding window) lets the query at
 *     position p see positions p-W+1 .. p.
 *   - the INT8 KV format ([897] description and "Regression and CUDA
 *     isolation" name INT8 KV beside FP8 and BF16, with no definition) is the
 *     symmetric per-row counterpart of the FP8 one: s = fl32(amax / 127),
 *     code = round-half-even(fl32(x / s)) clamped to [-127, 127], stored as a
 *     two's-complement byte; value = code * s.
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -fopenmp -ffp-contract=off.
 * No fast-math: fp32 divisions and products must be IEEE round-to-nearest.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#if !defined(FLT_EVAL_METHOD) || FLT_EVAL_METHOD != 0
#error "the oracle needs float expressions evaluated in float (FLT_EVAL_METHOD == 0)"
#endif

/* Largest head dim the oracle handles (stack arrays are sized by it). */
#define ORACLE_MAX_HEAD_DIM 256

/* ---------------------------------------------------------------- bf16 -- */

/* bf16 is the top half of an IEEE binary32; widening is exact. */
static float bf16_to_float(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round a binary32 to bf16, round-to-nearest, ties to even (finite inputs).
 * Dropping 16 low bits: add half an output ulp minus one, plus the output's
 * lowest kept bit so that an exact half rounds towards the even neighbour. */
static uint16_t float_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u); /* quiet NaN */
    uint32_t keep_lsb = (u >> 16) & 1u;
    u += 0x7fffu + keep_lsb;
    return (uint16_t)(u >> 16);
}

uint16_t oracle_f32_to_bf16(float f) { return float_to_bf16_rne(f); }
float oracle_bf16_to_f32(uint16_t b) { return bf16_to_float(b); }

/* ------------------------------------------------------------- E4M3FN -- */

/* [OFP8] decode of one code byte, exactly, as a double.  NaN for 0x7F/0xFF. */
double oracle_e4m3_decode(uint8_t c) {
    int sign = c >> 7;
    int e = (c >> 3) & 0xF;
    int m = c & 0x7;
    double mag;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);             /* subnormal: m * 2^-9 */
    else
        mag = ldexp(1.0 + m / 8.0, e - 7);      /* normal: 1.m * 2^(e-7) */
    return sign ? -mag : mag;
}

/* [OFP8] + saturation: encode a finite binary32 as E4M3FN, round to nearest
 * even, magnitudes at or above 448 saturate to 448 (code 0x7E | sign).
 *
 * Finite E4M3 magnitudes, listed by code, increase with the code: codes 0..8
 * are n * 2^-9 (n = 0..8; code 8 is 2^-6, the first normal), and in the binade
 * [2^E, 2^(E+1)) for E = -6..8 the codes are ((E+7) << 3) + (n - 8) for
 * magnitudes n * 2^(E-3), n = 8..15.  So rounding |y| to an integer multiple n
 * of the local grid step, ties to even n, and mapping n back to a code is the
 * round-to-nearest-even encoding; n reaching 16 lands on the next binade's
 * first code by the same formula. */
uint8_t oracle_e4m3_encode(float y) {
    uint8_t sign = signbit(y) ? 0x80 : 0x00;
    double a = fabs((double)y);
    double step, q, n, frac;
    int code, E, ex;
    if (a >= 448.0)
        return sign | 0x7E;
    if (a < ldexp(1.0, -6)) {
        step = ldexp(1.0, -9);
        E = -100; /* subnormal range: code == n */
    } else {
        (void)frexp(a, &ex); /* a = f * 2^ex, f in [0.5, 1) */
        E = ex - 1;          /* a in [2^E, 2^(E+1)) */
        step = ldexp(1.0, E - 3);
    }
    q = a / step; /* exact: division by a power of two */
    n = floor(q);
    frac = q - n;
    if (frac > 0.5 || (frac == 0.5 && fmod(n, 2.0) != 0.0))
        n += 1.0;
    if (E == -100)
        code = (int)n;
    else
        code = ((E + 7) << 3) + ((int)n - 8);
    if (code > 0x7E) /* cannot happen for a < 448; kept as a guard */
        code = 0x7E;
    return sign | (uint8_t)code;
}

/* --------------------------------------------------------------- INT8 -- */

/* Round a finite binary32 to the nearest integer, ties to even, clamped to
 * [-127, 127] (the symmetric INT8 KV format). */
int8_t oracle_int8_encode(float y) {
    double a = (double)y, n = floor(a), frac = a - n;
    if (frac > 0.5 || (frac == 0.5 && fmod(n, 2.0) != 0.0))
        n += 1.0;
    if (n > 127.0)
        n = 127.0;
    if (n < -127.0)
        n = -127.0;
    return (int8_t)n;
}

/* Value of an INT8 code byte (two's complement). */
double oracle_int8_decode(uint8_t c) { return (double)(int8_t)c; }

/* ---------------------------------------------------------- quantize -- */

/* KV code formats. */
#define ORACLE_FORMAT_E4M3 0
#define ORACLE_FORMAT_INT8 1

/* Quantize one row of D bf16 values ([853] "What changes": one FP32 scale
 * per physical K/V row; [280]: dynamic per-token / per-KV-head scale).
 *   amax = max |x|, s = fl32(amax / 448), c_d = encode(fl32(x_d / s)).
 * amax == 0 gives s = 0 and codes that keep the sign of each zero input. */
static void quantize_row(const uint16_t *x, int32_t D, uint8_t *codes, float *scale) {
    float xf[ORACLE_MAX_HEAD_DIM];
    float amax = 0.0f, s;
    int d;
    for (d = 0; d < D; ++d) {
        xf[d] = bf16_to_float(x[d]);
        if (fabsf(xf[d]) > amax)
            amax = fabsf(xf[d]);
    }
    s = amax / 448.0f;
    for (d = 0; d < D; ++d) {
        float yd = (amax == 0.0f) ? xf[d] : xf[d] / s;
        codes[d] = oracle_e4m3_encode(yd);
    }
    *scale = s;
}

/* The INT8 counterpart: amax = max |x|, s = fl32(amax / 127),
 * c_d = int8_encode(fl32(x_d / s)); amax == 0 gives s = 0 and zero codes. */
static void quantize_row_int8(const uint16_t *x, int32_t D, uint8_t *codes, float *scale) {
    float xf[ORACLE_MAX_HEAD_DIM];
    float amax = 0.0f, s;
    int d;
    for (d = 0; d < D; ++d) {
        xf[d] = bf16_to_float(x[d]);
        if (fabsf(xf[d]) > amax)
            amax = fabsf(xf[d]);
    }
    s = amax / 127.0f;
    for (d = 0; d < D; ++d)
        codes[d] = (uint8_t)((amax == 0.0f) ? 0 : oracle_int8_encode(xf[d] / s));
    *scale = s;
}

/* rows: [n_rows][head_dim] bf16 bits, contiguous.  codes: [n_rows][head_dim];
 * scales: [n_rows].  format: ORACLE_FORMAT_E4M3 or ORACLE_FORMAT_INT8.
 * head_dim in [1, ORACLE_MAX_HEAD_DIM]; returns 0, or -1 for an unsupported
 * head_dim or format. */
int32_t oracle_quantize_rows(const uint16_t *rows, int64_t n_rows, int32_t head_dim, int32_t format,
                             uint8_t *codes, float *scales) {
    int64_t r;
    if (head_dim <= 0 || head_dim > ORACLE_MAX_HEAD_DIM)
        return -1;
    if (format != ORACLE_FORMAT_E4M3 && format != ORACLE_FORMAT_INT8)
        return -1;
#pragma omp parallel for schedule(static)
    for (r = 0; r < n_rows; ++r) {
        if (format == ORACLE_FORMAT_INT8)
            quantize_row_int8(rows + r * head_dim, head_dim, codes + r * head_dim, scales + r);
        else
            quantize_row(rows + r * head_dim, head_dim, codes + r * head_dim, scales + r);
    }
    return 0;
}

/* Value table of one code format. */
static void code_values(int32_t format, double lut[256]) {
    int i;
    for (i = 0; i < 256; ++i)
        lut[i] = (format == ORACLE_FORMAT_INT8) ? oracle_int8_decode((uint8_t)i) : oracle_e4m3_decode((uint8_t)i);
}

/* --------------------------------------------------------- attention -- */

/* Decode attention over a page-size-1 FP8 pool ([853] "What changes"; [897]
 * description: BF16 query, GQA decode over FP8 rows with per-row scales).
 *
 * Pool layout (D = head_dim): codes of physical row r, KV head g start at
 *   k_codes + r * code_row_stride + g * D   (bytes),
 * scales at k_scales[r * scale_row_stride + g]; the same for V.
 * q: [batch][n_qrows][n_q_heads][D] bf16 bits.  table: [batch][table_stride].
 * out: [batch][n_qrows][n_q_heads][D] doubles.
 *
 * Request b holds positions 0 .. L-1 (L = seq_lens[b]) at rows table[b][t].
 * Its query row i (0 <= i < n_qrows) sits at position p = L - n_qrows + i and
 * sees positions t with lo <= t <= p, where lo = max(0, p - window + 1) for
 * window > 0 and lo = 0 otherwise.  For query head h (KV head
 * g = h / (n_q_heads / n_kv_heads)):
 *   khat_t = decode(k code) * k_scale,  vhat_t = decode(v code) * v_scale (fp64)
 *   z_t    = sm_scale * sum_d q_d * khat_t[d]
 *   out    = sum_t exp(z_t - max z) vhat_t / sum_t exp(z_t - max z)
 * with decode the E4M3FN or the INT8 value of a code byte (`format`).
 * A query row that sees no position (p < 0) gets an all-zero output.
 * Returns 0, or -1 for an unsupported head_dim or format. */
int32_t oracle_decode_attention(const uint16_t *q, int32_t batch, int32_t n_qrows, int32_t n_q_heads,
                                int32_t n_kv_heads, int32_t head_dim, int32_t format,
                                const uint8_t *k_codes, const uint8_t *v_codes,
                                const float *k_scales, const float *v_scales,
                                int64_t code_row_stride, int64_t scale_row_stride,
                                const int32_t *table, int64_t table_stride, const int32_t *seq_lens,
                                int32_t window, float sm_scale, double *out) {
    const int32_t D = head_dim;
    int32_t group = n_q_heads / n_kv_heads;
    int64_t job;
    double lut[256];
    if (D <= 0 || D > ORACLE_MAX_HEAD_DIM)
        return -1;
    if (format != ORACLE_FORMAT_E4M3 && format != ORACLE_FORMAT_INT8)
        return -1;
    code_values(format, lut);

#pragma omp parallel for schedule(dynamic, 1)
    for (job = 0; job < (int64_t)batch * n_qrows * n_q_heads; ++job) {
        int32_t h = (int32_t)(job % n_q_heads);
        int32_t qi = (int32_t)((job / n_q_heads) % n_qrows);
        int32_t b = (int32_t)(job / ((int64_t)n_q_heads * n_qrows));
        int32_t g = h / group;
        int64_t p = (int64_t)seq_lens[b] - n_qrows + qi, lo = 0, t;
        double qd[ORACLE_MAX_HEAD_DIM], acc[ORACLE_MAX_HEAD_DIM];
        double *z, zmax = -INFINITY, denom = 0.0;
        double *o = out + job * D;
        int d;
        if (window > 0 && p - window + 1 > 0)
            lo = p - window + 1;
        for (d = 0; d < D; ++d) {
            qd[d] = (double)bf16_to_float(q[job * D + d]);
            acc[d] = 0.0;
        }
        if (p < 0) {
            for (d = 0; d < D; ++d)
                o[d] = 0.0;
            continue;
        }
        z = (double *)malloc((size_t)(p - lo + 1) * sizeof(double));
        for (t = lo; t <= p; ++t) {
            int64_t row = table[(int64_t)b * table_stride + t];
            const uint8_t *kc = k_codes + row * code_row_stride + (int64_t)g * D;
            double ks = (double)k_scales[row * scale_row_stride + g];
            double dot = 0.0;
            for (d = 0; d < D; ++d)
                dot += qd[d] * (lut[kc[d]] * ks);
            z[t - lo] = dot * (double)sm_scale;
            if (z[t - lo] > zmax)
                zmax = z[t - lo];
        }
        for (t = lo; t <= p; ++t) {
            int64_t row = table[(int64_t)b * table_stride + t];
            const uint8_t *vc = v_codes + row * code_row_stride + (int64_t)g * D;
            double vs = (double)v_scales[row * scale_row_stride + g];
            double w = exp(z[t - lo] - zmax);
            denom += w;
            for (d = 0; d < D; ++d)
                acc[d] += w * (lut[vc[d]] * vs);
        }
        for (d = 0; d < D; ++d)
            o[d] = acc[d] / denom;
        free(z);
    }
    return 0;
}

/* --------------------------------------------------------- prefill -- */

/* Rebuild historical FP8 rows as bf16 ([853] "What changes": historical FP8
 * rows are reconstructed once per layer into one shared BF16 workspace).
 * ws[j][g][d] = bf16_rne(fl32(decode(code) * scale)) for pool row rows[j], with
 * decode the E4M3FN or INT8 value of the code (`format`).
 * ws: [n_rows][n_kv_heads][head_dim] bf16 bits. */
void oracle_reconstruct(const uint8_t *codes, const float *scales, int64_t code_row_stride,
                        int64_t scale_row_stride, int32_t n_kv_heads, int32_t head_dim, int32_t format,
                        const int32_t *rows, int64_t n_rows, uint16_t *ws) {
    int64_t j;
    double lut[256];
    code_values(format, lut);
#pragma omp parallel for schedule(static)
    for (j = 0; j < n_rows; ++j) {
        int64_t row = rows[j];
        int32_t g;
        int d;
        for (g = 0; g < n_kv_heads; ++g) {
            const uint8_t *c = codes + row * code_row_stride + (int64_t)g * head_dim;
            float s = scales[row * scale_row_stride + g];
            uint16_t *w = ws + (j * n_kv_heads + g) * head_dim;
            for (d = 0; d < head_dim; ++d) {
                float v = (float)lut[c[d]] * s; /* exact decode, one fp32 rounding */
                w[d] = float_to_bf16_rne(v);
            }
        }
    }
}

/* Prefill attention runs at D = 128, the head dim of the pages' prefill
 * measurements. */
#define ORACLE_PREFILL_HEAD_DIM 128

/* Chunked-prefill attention ([853] "What changes": the current chunk's K/V stay
 * BF16; historical rows come from the BF16 workspace).
 * Keys/values for chunk query i: ws rows 0..n_prefix-1, then chunk rows 0..i.
 * q: [n_chunk][n_q_heads][128]; ws_k/ws_v: [n_prefix][n_kv_heads][128];
 * k_cur/v_cur: [n_chunk][n_kv_heads][128]; all bf16 bits.
 * Only the queries listed in q_idx[0..n_q) are evaluated; out: [n_q][n_q_heads][128]. */
void oracle_prefill_attention(const uint16_t *q, const uint16_t *ws_k, const uint16_t *ws_v,
                              const uint16_t *k_cur, const uint16_t *v_cur, int32_t n_prefix,
                              int32_t n_chunk, int32_t n_q_heads, int32_t n_kv_heads, float sm_scale,
                              const int32_t *q_idx, int32_t n_q, double *out) {
    int32_t group = n_q_heads / n_kv_heads;
    int64_t job;
    (void)n_chunk;
#pragma omp parallel for schedule(dynamic, 1)
    for (job = 0; job < (int64_t)n_q * n_q_heads; ++job) {
        int32_t qi = (int32_t)(job / n_q_heads), h = (int32_t)(job % n_q_heads);
        int32_t i = q_idx[qi], g = h / group;
        int64_t n_keys = (int64_t)n_prefix + i + 1, u;
        double qd[ORACLE_PREFILL_HEAD_DIM], acc[ORACLE_PREFILL_HEAD_DIM];
        double *z = (double *)malloc((size_t)n_keys * sizeof(double));
        double zmax = -INFINITY, denom = 0.0;
        double *o = out + job * ORACLE_PREFILL_HEAD_DIM;
        int d;
        for (d = 0; d < ORACLE_PREFILL_HEAD_DIM; ++d) {
            qd[d] = (double)bf16_to_float(q[((int64_t)i * n_q_heads + h) * ORACLE_PREFILL_HEAD_DIM + d]);
            acc[d] = 0.0;
        }
        for (u = 0; u < n_keys; ++u) {
            const uint16_t *k = (u < n_prefix)
                ? ws_k + (u * n_kv_heads + g) * ORACLE_PREFILL_HEAD_DIM
                : k_cur + ((u - n_prefix) * n_kv_heads + g) * ORACLE_PREFILL_HEAD_DIM;
            double dot = 0.0;
            for (d = 0; d < ORACLE_PREFILL_HEAD_DIM; ++d)
                dot += qd[d] * (double)bf16_to_float(k[d]);
            z[u] = dot * (double)sm_scale;
            if (z[u] > zmax)
                zmax = z[u];
        }
        for (u = 0; u < n_keys; ++u) {
            const uint16_t *v = (u < n_prefix)
                ? ws_v + (u * n_kv_heads + g) * ORACLE_PREFILL_HEAD_DIM
                : v_cur + ((u - n_prefix) * n_kv_heads + g) * ORACLE_PREFILL_HEAD_DIM;
            double w = exp(z[u] - zmax);
            denom += w;
            for (d = 0; d < ORACLE_PREFILL_HEAD_DIM; ++d)
                acc[d] += w * (double)bf16_to_float(v[d]);
        }
        for (d = 0; d < ORACLE_PREFILL_HEAD_DIM; ++d)
            o[d] = acc[d] / denom;
        free(z);
    }
}

/* ------------------------------------------------------ accounting -- */

/* Bytes one token occupies across all layers ([853] "Validation" and
 * "Follow-up model/workload search"): FP8 stores, per layer, K and V, per KV
 * head, head_dim code bytes plus one 4-byte scale; BF16 stores 2 bytes per
 * element. */
int64_t oracle_fp8_bytes_per_token(int32_t n_layers, int32_t n_kv_heads, int32_t head_dim) {
    return (int64_t)n_layers * 2 * n_kv_heads * ((int64_t)head_dim + 4);
}

int64_t oracle_bf16_bytes_per_token(int32_t n_layers, int32_t n_kv_heads, int32_t head_dim) {
    return (int64_t)n_layers * 2 * n_kv_heads * (int64_t)head_dim * 2;
}

/* One layer of K and V in BF16 for every pool row: the shared prefill workspace. */
int64_t oracle_bf16_workspace_bytes(int64_t n_rows, int32_t n_kv_heads, int32_t head_dim) {
    return n_rows * 2 * n_kv_heads * (int64_t)head_dim * 2;
}

int32_t oracle_num_threads(void) {
#ifdef _OPENMP
    return (int32_t)omp_get_max_threads();
#else
    return 1;
#endif
}

/* Host threads for the following calls from this thread (timing runs only;
 * results do not depend on it). */
void oracle_set_num_threads(int32_t n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
