/*
 * fp8kv.h -- C ABI of libfp8kv.so: an FP8 (OCP E4M3FN) per-row KV cache and the
 * GQA attention that reads it, for AMD Instinct MI355X (gfx950).
 *
 * The operations follow FreeToken PR #853 "opt-in FP8 KV cache", section "What
 * changes": each physical K/V row stores E4M3 code bytes plus its own FP32
 * scale; decode attention reads those rows directly; prefill rebuilds the
 * historical FP8 rows once per layer into one shared BF16 workspace while the
 * current chunk's K/V stay BF16.  FreeToken PR #897 "perf(attention): add packed
 * fp8 kv reads on gfx1201" (description; "Fresh R9700 stage-1 A/B") fixes the
 * decode case: BF16 query, head dim 128, GQA 4/8, page size 1 with randomized
 * physical slots, a split-K first stage and a merge kernel; its section
 * "Regression and CUDA isolation" widens the decode matrix to head dim 256,
 * 1/3/8 query rows per request and an odd sliding window.
 *
 * Entry points: fp8kv_quantize_rows (quantize-on-write); fp8kv_decode_attn and
 * its two stages fp8kv_decode_stage1 / fp8kv_decode_merge (and
 * fp8kv_decode_stage1_valu, stage 1 on the vector units for comparison);
 * fp8kv_decode_attn_rows
 * (several query rows, sliding window); fp8kv_decode_attn_append,
 * fp8kv_decode_attn_append_window and fp8kv_decode_attn_rows_append (a decode
 * step with its new tokens quantized on write in the same call);
 * fp8kv_decode_attn_append_noalloc (the same step without a caller workspace);
 * fp8kv_prefill_attn (reconstruct + causal chunk attention) and
 * fp8kv_prefill_attn_workspace (the attention over an already rebuilt
 * workspace);
 * fp8kv_decode_workspace_bytes and fp8kv_status_string.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    allocates nothing, copies nothing between host and device and never
 *    synchronizes.  Work is enqueued on `stream` (a hipStream_t; NULL = the
 *    null stream) and the call returns immediately, so calls may be captured
 *    into a HIP graph.
 *  - bf16 tensors are passed as uint16_t bit patterns.
 *  - Every argument that can be checked without reading device memory is
 *    checked on the host before anything is enqueued; on error nothing is
 *    launched and nothing is written.  Device-resident contents (row indices in
 *    tables and slot lists, sequence lengths, finiteness of inputs) are
 *    preconditions: an out-of-range row index is undefined behaviour.
 *  - sm_scale (the softmax scale of the attention calls) must be finite and
 *    greater than zero; anything else returns FP8KV_ERR_INVALID_ARG.
 *  - Functions are stateless apart from a per-device cache of the compute-unit
 *    count; they are thread-safe and may run concurrently on different streams
 *    as long as their output buffers do not overlap.
 *  - The library runs on gfx950 only; on other devices calls return
 *    FP8KV_ERR_UNSUPPORTED.
 */
#ifndef FP8KV_H
#define FP8KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Head dimensions: pools, quantize-on-write and decode take either; the
 * prefill path runs at FP8KV_HEAD_DIM. */
#define FP8KV_HEAD_DIM 128
#define FP8KV_HEAD_DIM_256 256
/* Largest finite E4M3FN magnitude; a row's scale is amax / FP8KV_E4M3_MAX. */
#define FP8KV_E4M3_MAX 448.0f
/* Upper bound on decode key-splits per (request, KV head). */
#define FP8KV_MAX_SPLITS 256
/* Upper bound on query rows per request in one decode call. */
#define FP8KV_MAX_QUERY_ROWS 8
/* Upper bound on requests per decode call (times ceil(G * n_qrows / 32) for
 * several query rows): they share one launch dimension. */
#define FP8KV_MAX_DECODE_GROUPS 65535
/* Bytes of the per-device array that holds the split partials of
 * fp8kv_decode_attn_append_noalloc (32 MiB). */
#define FP8KV_NOALLOC_SCRATCH_BYTES 33554432
/* Code formats of a pool (fp8kv_pool_layer.code_format). */
#define FP8KV_CODE_E4M3 0 /* OCP E4M3FN, scale amax / 448 */
#define FP8KV_CODE_INT8 1 /* symmetric INT8, scale amax / 127 */

typedef enum fp8kv_status {
    FP8KV_OK = 0,
    FP8KV_ERR_INVALID_ARG = 1, /* null pointer, non-positive or inconsistent size */
    FP8KV_ERR_UNSUPPORTED = 2, /* head_dim not 128/256 (128 for prefill), code format, GQA ratio, not gfx950 */
    FP8KV_ERR_ALIGNMENT = 3,   /* a base pointer or stride breaks the alignment contract */
    FP8KV_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required */
    FP8KV_ERR_HIP = 5          /* the HIP runtime rejected a launch or a query */
} fp8kv_status;

/*
 * One layer of the page-size-1 FP8 row pool (FreeToken PR #853, "What
 * changes": every physical K/V row holds E4M3 code bytes plus its own FP32
 * scale; issue #280, "Current proof-of-concept limitations": dynamic scales per
 * token and per KV head).
 *
 * Physical row r, KV head g, with D = head_dim (128 or 256):
 *   K codes   k_codes  + r * code_row_stride + g * D     (D bytes)
 *   V codes   v_codes  + r * code_row_stride + g * D     (D bytes)
 *   K scale   k_scales[r * scale_row_stride + g]         (fp32)
 *   V scale   v_scales[r * scale_row_stride + g]         (fp32)
 * Value of element d: decode(code[d]) * scale, where decode is the OCP E4M3FN
 * value of the byte (code_format FP8KV_CODE_E4M3) or the byte read as a
 * two's-complement integer (FP8KV_CODE_INT8: the pages list INT8 KV beside
 * FP8, FreeToken PR #897 description and "Regression and CUDA isolation";
 * this library takes it as the symmetric per-row counterpart, scale
 * amax / 127, codes in [-127, 127]).
 *
 * Alignment contract (FreeToken PR #897 description: packed reads need
 * 16-byte-aligned bases and row/head strides): k_codes, v_codes and
 * code_row_stride are multiples of 16 bytes; k_scales and v_scales are 4-byte
 * aligned.  code_row_stride >= n_kv_heads * D and scale_row_stride >=
 * n_kv_heads.  Strides let the four arrays be separate allocations or
 * interleave inside one per-row record.
 *
 * When k_codes, v_codes and code_row_stride are also multiples of 128 bytes,
 * every KV head's code rows fill whole 128-byte lines that no other KV head
 * reads, and the decode calls read the codes with non-temporal loads: faster
 * for a pool read from HBM (a model's layers, each read once per token),
 * slower for one read over and over from the Infinity Cache.  A per-row
 * record of 2 * n_kv_heads * (D + 4) bytes padded to a multiple of 128 (1,152
 * bytes for 4 KV heads, D = 128) gets this; so do separate arrays with
 * 128-byte-aligned bases.  Results are the same either way.
 */
typedef struct fp8kv_pool_layer {
    uint8_t *k_codes;
    uint8_t *v_codes;
    float *k_scales;
    float *v_scales;
    int64_t num_rows;         /* physical rows in the pool */
    int32_t n_kv_heads;       /* KV heads per row */
    int32_t head_dim;         /* FP8KV_HEAD_DIM or FP8KV_HEAD_DIM_256 */
    int64_t code_row_stride;  /* bytes between rows of k_codes / v_codes */
    int64_t scale_row_stride; /* floats between rows of k_scales / v_scales */
    int32_t code_format;      /* FP8KV_CODE_E4M3 (0) or FP8KV_CODE_INT8 */
    int32_t reserved;         /* must be 0 */
} fp8kv_pool_layer;

/*
 * fp8kv_quantize_rows -- quantize-on-write of new K/V rows (FreeToken PR #853,
 * "Follow-up model/workload search": the FP8 path quantizes each new K/V row;
 * "What changes": each row stores E4M3 codes plus its own FP32 scale).
 *
 * For token t in [0, n_tokens), KV head g, separately for K and V, with x the
 * D = pool->head_dim bf16 values at k + t * src_token_stride + g * D (resp. v):
 *   amax = max_d |x_d|;   s = fl32(amax / 448)   (IEEE fp32 division)
 *   code_d = E4M3FN round-to-nearest-even of fl32(x_d / s), saturated to +-448
 *   (a row with amax == 0 stores s = 0 and codes +0 / -0 following x_d's sign)
 * and stores the codes and s at physical row slots[t].  An INT8 pool stores
 *   s = fl32(amax / 127),  code_d = round-half-even(fl32(x_d / s)) clamped to
 *   [-127, 127]  (amax == 0: s = 0, codes 0).
 *
 * k, v:            device bf16 [n_tokens][n_kv_heads][D] with token stride
 *                  src_token_stride elements (>= n_kv_heads*D, a multiple of
 *                  8); bases 16-byte aligned.
 * slots:           device int32 [n_tokens], each in [0, pool->num_rows); slots
 *                  must be distinct within one call.  An out-of-range slot is
 *                  clamped to num_rows - 1 (never an access outside the pool).
 * n_tokens:        >= 0 (0 is a no-op).
 * Errors: INVALID_ARG (null pointer, bad sizes), UNSUPPORTED, ALIGNMENT, HIP.
 */
fp8kv_status fp8kv_quantize_rows(const fp8kv_pool_layer *pool, const uint16_t *k, const uint16_t *v,
                                 int64_t src_token_stride, const int32_t *slots, int32_t n_tokens,
                                 void *stream);

/*
 * Bytes of device workspace the decode calls need for `n_queries` query rows
 * (batch * n_qrows; batch for the one-row calls) of `n_q_heads` query heads
 * of dimension `head_dim` with at most `max_splits` splits per request
 * (0 = FP8KV_MAX_SPLITS): a 256-byte header, then one fp32 output vector and
 * one log-sum-exp per query row, query head and split slot.  Returns 0 for
 * invalid arguments.
 */
size_t fp8kv_decode_workspace_bytes(int32_t n_queries, int32_t n_q_heads, int32_t head_dim, int32_t max_splits);

/*
 * fp8kv_decode_attn -- one-token-per-request GQA attention over the FP8 pool
 * (FreeToken PR #897 description and "Fresh R9700 stage-1 A/B": BF16 query,
 * D = 128, GQA 4/8, page size 1, split-K stage 1 followed by a merge kernel;
 * "Regression and CUDA isolation": D = 256 as well; PR #853 "What changes":
 * rows hold E4M3 codes and per-row FP32 scales).  D = pool->head_dim.
 *
 * For request b and query head h, with G = n_q_heads / n_kv_heads, KV head
 * g = h / G, L = seq_lens[b] and rows r_t = row_table[b * table_stride + t]:
 *   z_t   = sm_scale * sum_d q[b][h][d] * decode(Kcode[r_t][g][d]) * k_scale[r_t][g]
 *   out[b][h] = sum_t softmax(z)_t * decode(Vcode[r_t][g]) * v_scale[r_t][g]
 * rounded to bf16.  A request with L == 0 gets zeros.
 *
 * Equivalent to fp8kv_decode_stage1 followed by fp8kv_decode_merge on the same
 * stream.  Stage 1 splits each request's rows into at most `max_splits`
 * (0 = chosen from the device's compute-unit count and max_seq_len) ranges and
 * writes one partial per (request, query head, split) into `workspace`; the
 * merge combines them by log-sum-exp.  Results agree to rounding for every
 * split count.
 *
 * Timing depends on the data in one case: stage 1 measures each key's weight
 * against the largest score among the first keys it reads (D = 128), and
 * when a later score is so much larger that a weight or a sum overflows
 * (about 128 powers of two in exp2 units), that part of the keys is read and
 * summed a second time with a running maximum.  The result is the same up to
 * rounding either way.  The prefill attention does the same per workgroup.
 *
 * q:            device bf16 [batch][n_q_heads][D], contiguous, 16-byte aligned
 *               (D = pool->head_dim).
 * row_table:    device int32, row b at row_table + b * table_stride; all
 *               batch * table_stride entries must be readable (the kernels
 *               read entries up to max(max_seq_len, 1) of a row before the
 *               length is known).  Entries below seq_lens[b] name the
 *               request's rows.  Entries
 *               in [seq_lens[b], max_seq_len) (padding) are read and masked
 *               out (weight 0).  Every kernel clamps a row index to
 *               [0, num_rows) before using it (an out-of-range entry reads
 *               row num_rows - 1, never memory outside the pool), and the
 *               row an entry resolves to must hold finite codes and scales
 *               (written by fp8kv_quantize_rows, or zero-filled): a masked
 *               key has weight exactly 0, which a NaN value would still
 *               turn into NaN.
 * seq_lens:     device int32 [batch], each in [0, max_seq_len].
 * max_seq_len:  host-side upper bound on seq_lens (sizes the launch), >= 0,
 *               <= table_stride.
 * n_q_heads:    a multiple of pool->n_kv_heads with G in {1, 2, 4, 8, 16}.
 * batch:        1 .. FP8KV_MAX_DECODE_GROUPS (one launch dimension holds the
 *               requests; for fp8kv_decode_attn_rows it holds the requests
 *               times ceil(G * n_qrows / 32), which must not exceed it).
 * workspace:    device, 256-byte aligned, >= fp8kv_decode_workspace_bytes(
 *               batch, n_q_heads, D, max_splits) bytes; contents are scratch.
 * out:          device bf16 [batch][n_q_heads][D], 16-byte aligned.
 * Errors: INVALID_ARG, UNSUPPORTED (G, head_dim, batch over the limit),
 *         ALIGNMENT, WORKSPACE, HIP.
 */
fp8kv_status fp8kv_decode_attn(const fp8kv_pool_layer *pool, const uint16_t *q, int32_t batch,
                               int32_t n_q_heads, const int32_t *row_table, int64_t table_stride,
                               const int32_t *seq_lens, int32_t max_seq_len, float sm_scale,
                               int32_t max_splits, void *workspace, size_t workspace_bytes,
                               uint16_t *out, void *stream);

/*
 * fp8kv_decode_stage1 -- the split-K first stage of fp8kv_decode_attn alone
 * (FreeToken PR #897, "Fresh R9700 stage-1 A/B": stage 1 is timed apart from
 * the merge kernel).  Same arguments and checks as fp8kv_decode_attn without
 * `out`; writes the partials and the split count into `workspace`.
 */
fp8kv_status fp8kv_decode_stage1(const fp8kv_pool_layer *pool, const uint16_t *q, int32_t batch,
                                 int32_t n_q_heads, const int32_t *row_table, int64_t table_stride,
                                 const int32_t *seq_lens, int32_t max_seq_len, float sm_scale,
                                 int32_t max_splits, void *workspace, size_t workspace_bytes,
                                 void *stream);

/*
 * fp8kv_decode_stage1_valu -- fp8kv_decode_stage1 computed without matrix
 * instructions (plain fp32 vector FMAs: one key per lane for the QK^T dot
 * products, two output elements per lane for P*V), on the same grid and into
 * the same partials, so fp8kv_decode_merge combines it.  It exists to measure
 * the decode contraction on the vector units against the bf16 MFMA path of
 * fp8kv_decode_stage1 on the same inputs (FreeToken PR #897 description: the
 * RDNA4 reader widens FP8 for the existing matrix math; which unit wins is a
 * property of the hardware).  Same arguments, checks and errors as
 * fp8kv_decode_stage1; head_dim 128 and E4M3 pools only (others return
 * FP8KV_ERR_UNSUPPORTED).
 */
fp8kv_status fp8kv_decode_stage1_valu(const fp8kv_pool_layer *pool, const uint16_t *q, int32_t batch,
                                      int32_t n_q_heads, const int32_t *row_table, int64_t table_stride,
                                      const int32_t *seq_lens, int32_t max_seq_len, float sm_scale,
                                      int32_t max_splits, void *workspace, size_t workspace_bytes,
                                      void *stream);

/*
 * fp8kv_decode_merge -- the merge (stage 2) of the decode calls: combines the
 * partials a preceding fp8kv_decode_stage1 on the same stream wrote into
 * `workspace` (n_queries = its batch; the same n_q_heads, head dim and
 * max_splits) by log-sum-exp and writes bf16 out[n_queries][n_q_heads][head_dim].
 * The split count comes from the workspace header that stage 1 wrote; it is
 * clamped to the workspace's split capacity, so a workspace no stage 1 wrote
 * gives meaningless output but no access outside the workspace (a header
 * holding 0 or less gives all-zero output).
 * Errors: INVALID_ARG, UNSUPPORTED (head_dim), ALIGNMENT, WORKSPACE, HIP.
 */
fp8kv_status fp8kv_decode_merge(int32_t n_queries, int32_t n_q_heads, int32_t head_dim, int32_t max_splits,
                                const void *workspace, size_t workspace_bytes, uint16_t *out,
                                void *stream);

/*
 * fp8kv_decode_attn_rows -- decode attention for several query rows per
 * request and an optional sliding key window (FreeToken PR #897 description:
 * the multi-row decode of #900 runs up to 8 query rows per request; "Regression
 * and CUDA isolation": 1/3/8 query rows and an odd sliding window are part of
 * the qualified matrix).
 *
 * Request b holds positions 0 .. L-1 (L = seq_lens[b]) at rows
 * row_table[b * table_stride + t].  Its query row i (0 <= i < n_qrows) sits at
 * position p = L - n_qrows + i (its own K/V are already in the pool) and
 * attends causally to positions lo .. p, lo = max(0, p - window + 1) when
 * window > 0 and lo = 0 when window == 0; a row with p < 0 gets zeros.  Each
 * row is fp8kv_decode_attn's formula over its own positions.  n_qrows == 1
 * with window == 0 is fp8kv_decode_attn.
 *
 * Rows share the reads of the K/V codes: the G * n_qrows (query row, head)
 * pairs of a KV head are the columns of the MFMA tiles, up to 64 per
 * workgroup at D = 128 and 32 at D = 256 (wider shapes run more workgroups
 * over the same rows).
 *
 * q, out:       device bf16 [batch][n_qrows][n_q_heads][D], 16-byte aligned.
 * n_qrows:      1 .. FP8KV_MAX_QUERY_ROWS.
 * window:       >= 0 (0 = no window).
 * workspace:    >= fp8kv_decode_workspace_bytes(batch * n_qrows, n_q_heads,
 *               D, max_splits) bytes.
 * Other arguments and the errors are those of fp8kv_decode_attn.
 */
fp8kv_status fp8kv_decode_attn_rows(const fp8kv_pool_layer *pool, const uint16_t *q, int32_t batch, int32_t n_qrows,
                                    int32_t n_q_heads, const int32_t *row_table, int64_t table_stride,
                                    const int32_t *seq_lens, int32_t max_seq_len, int32_t window, float sm_scale,
                                    int32_t max_splits, void *workspace, size_t workspace_bytes, uint16_t *out,
                                    void *stream);

/*
 * fp8kv_decode_attn_append -- one decode step with the new token's
 * quantize-on-write folded in (FreeToken PR #853 "Follow-up model/workload
 * search": on the FP8 path every new K/V row is quantized as it is written;
 * PR #897 description: the decode reader then attends over the pool).
 *
 * For each request b the new token sits at position p_b = seq_lens[b] - 1,
 * and its pool row is new_slots[b] (== row_table[b * table_stride + p_b]).
 * The call has the effect of
 *   fp8kv_quantize_rows(pool, k_new, v_new, new_token_stride, new_slots, batch)
 * followed by fp8kv_decode_attn with the same arguments: the token's codes and
 * scales land in its row bit for bit as fp8kv_quantize_rows would write them,
 * and `out` is attention over positions [0, seq_lens[b]) including the token.
 * The token's row is never read back: stage 1 covers [0, p_b), and the token
 * is quantized and added as one more key inside the call, which saves a launch
 * per step -- by stage 1 (its first split's workgroup, folded into that
 * split's partial) when D = 128 and the call's splits fit one round of
 * workgroups, otherwise by the merge as a single-key partial.
 *
 * k_new, v_new:      device bf16, token b at k_new + b * new_token_stride,
 *                    [n_kv_heads][D] each; 16-byte aligned, stride a
 *                    multiple of 8 elements and >= n_kv_heads * D.
 * new_slots:         device int32 [batch], 4-byte aligned: physical rows of
 *                    `pool`, distinct between requests, named by no position
 *                    below p_b of any request (clamped like table entries).
 * seq_lens:          device int32 [batch], each in [1, max_seq_len].
 * row_table:         as for fp8kv_decode_attn.
 * Other arguments, the workspace and the errors are those of
 * fp8kv_decode_attn; max_seq_len must be >= 1.
 */
fp8kv_status fp8kv_decode_attn_append(const fp8kv_pool_layer *pool, const uint16_t *q, int32_t batch,
                                      int32_t n_q_heads, const uint16_t *k_new, const uint16_t *v_new,
                                      int64_t new_token_stride, const int32_t *new_slots,
                                      const int32_t *row_table,
                                      int64_t table_stride, const int32_t *seq_lens, int32_t max_seq_len,
                                      float sm_scale, int32_t max_splits, void *workspace,
                                      size_t workspace_bytes, uint16_t *out, void *stream);

/*
 * fp8kv_decode_attn_append_noalloc -- fp8kv_decode_attn_append for callers
 * that cannot allocate device memory or pass a workspace (code under HIP
 * graph capture that must not allocate, tight serving loops, harnesses that
 * forbid hipMalloc): the same computation, the same kernels and the same
 * results bit for bit, with the split partials kept in a fixed array of
 * FP8KV_NOALLOC_SCRATCH_BYTES bytes inside the library instead of a caller
 * workspace.  The call allocates nothing and frees nothing.
 *
 * The array exists once per GPU the library runs on and is held until the
 * process ends.  Every call on a GPU uses that GPU's array, which keeps the
 * previous call's contents (nothing in it needs to start at zero: stage 1
 * writes every partial the merge reads).  Calls that overlap in time on one
 * GPU -- on different streams, or from different threads -- race on the
 * array and must be serialized by the caller.
 *
 * The partials need 256 + batch * n_q_heads * S * (head_dim + 1) * 4 bytes,
 * with S the split count the call chooses (at most max_splits, 0 = chosen
 * from the device; 64 for one 32K-context request on MI355X); a call that
 * needs more than FP8KV_NOALLOC_SCRATCH_BYTES returns FP8KV_ERR_WORKSPACE
 * before launching anything.
 *
 * Arguments and the other errors are those of fp8kv_decode_attn_append
 * without `workspace` / `workspace_bytes`.
 */
fp8kv_status fp8kv_decode_attn_append_noalloc(const fp8kv_pool_layer *pool, const uint16_t *q, int32_t batch,
                                              int32_t n_q_heads, const uint16_t *k_new, const uint16_t *v_new,
                                              int64_t new_token_stride, const int32_t *new_slots,
                                              const int32_t *row_table, int64_t table_stride,
                                              const int32_t *seq_lens, int32_t max_seq_len, float sm_scale,
                                              int32_t max_splits, uint16_t *out, void *stream);

/*
 * fp8kv_decode_attn_append_window -- fp8kv_decode_attn_append with a sliding
 * key window (FreeToken PR #897, "Regression and CUDA isolation": an odd
 * sliding window is among the decode cases): the new token at p_b attends to
 * positions max(0, p_b - window + 1) .. p_b, itself included; window == 0 means
 * no window and is exactly fp8kv_decode_attn_append.  The effect is that of
 *   fp8kv_quantize_rows(pool, k_new, v_new, new_token_stride, new_slots, batch)
 * followed by fp8kv_decode_attn_rows with one query row and the same window.
 *
 * window:       >= 0.  Other arguments, the workspace and the errors are
 *               those of fp8kv_decode_attn_append.
 */
fp8kv_status fp8kv_decode_attn_append_window(const fp8kv_pool_layer *pool, const uint16_t *q, int32_t batch,
                                             int32_t n_q_heads, const uint16_t *k_new, const uint16_t *v_new,
                                             int64_t new_token_stride, const int32_t *new_slots,
                                             const int32_t *row_table, int64_t table_stride,
                                             const int32_t *seq_lens, int32_t max_seq_len, int32_t window,
                                             float sm_scale, int32_t max_splits, void *workspace,
                                             size_t workspace_bytes, uint16_t *out, void *stream);

/*
 * fp8kv_decode_attn_rows_append -- fp8kv_decode_attn_rows with the new tokens'
 * quantize-on-write folded in: each request's last n_qrows positions are new
 * tokens (FreeToken PR #897 description: #900's multi-row decode of up to 8
 * query rows per request), written to their rows and attended in one call.
 *
 * Request b's new token j (0 <= j < n_qrows) sits at position
 * p_bj = seq_lens[b] - n_qrows + j; its bf16 K/V are at
 * k_new / v_new + (b * n_qrows + j) * new_token_stride ([n_kv_heads][D]) and
 * its pool row is new_slots[b * n_qrows + j] (== row_table[b][p_bj]).  The
 * call has the effect of
 *   fp8kv_quantize_rows(pool, k_new, v_new, new_token_stride, new_slots,
 *                       batch * n_qrows)
 * followed by fp8kv_decode_attn_rows with the same arguments and window: the
 * codes and scales land bit for bit as fp8kv_quantize_rows writes them, and
 * query row j of request b attends causally (and within the window) over
 * positions up to p_bj.  Stage 1 covers the cached positions below the new
 * tokens; the merge quantizes the new tokens and adds the visible ones.
 *
 * q, out:       device bf16 [batch][n_qrows][n_q_heads][D], 16-byte aligned.
 * seq_lens:     device int32 [batch], each in [n_qrows, max_seq_len].
 * new_slots:    device int32 [batch * n_qrows], 4-byte aligned, distinct, not
 *               named by any cached position (clamped like table entries).
 * n_qrows:      1 .. FP8KV_MAX_QUERY_ROWS; max_seq_len >= n_qrows.
 * Other arguments, the workspace (fp8kv_decode_workspace_bytes(batch *
 * n_qrows, ...)) and the errors are those of fp8kv_decode_attn_rows and
 * fp8kv_decode_attn_append.
 */
fp8kv_status fp8kv_decode_attn_rows_append(const fp8kv_pool_layer *pool, const uint16_t *q, int32_t batch,
                                           int32_t n_qrows, int32_t n_q_heads, const uint16_t *k_new,
                                           const uint16_t *v_new, int64_t new_token_stride,
                                           const int32_t *new_slots, const int32_t *row_table,
                                           int64_t table_stride, const int32_t *seq_lens, int32_t max_seq_len,
                                           int32_t window, float sm_scale, int32_t max_splits, void *workspace,
                                           size_t workspace_bytes, uint16_t *out, void *stream);

/*
 * fp8kv_prefill_attn -- attention of one prefill chunk over historical FP8 rows
 * of a pool with head_dim == 128
 * (FreeToken PR #853, "What changes": the prefill path reconstructs historical
 * FP8 rows once per layer into one shared BF16 workspace; current-chunk K/V
 * remain BF16; "Paired end-to-end A/B": the 8K historical-prefix + 8K
 * new-token operator).
 *
 * Step 1 (reconstruct): for j in [0, n_prefix), KV head g, d in [0, 128):
 *   ws_k[j][g][d] = bf16_rne(fl32(decode(Kcode[prefix_rows[j]][g][d]) * k_scale))
 *   and the same for ws_v from the V codes and scales.
 * Step 2 (attention): chunk query i (absolute position n_prefix + i) attends
 *   to keys/values [ws rows 0..n_prefix-1 ; chunk rows 0..i] (causal), with
 *   KV head g = h / (n_q_heads / n_kv_heads) and softmax scale sm_scale;
 *   out[i][h] is rounded to bf16.
 * The chunk's own K/V are NOT written to the pool here; quantize them with
 * fp8kv_quantize_rows (before or after: the slots must not be prefix rows).
 *
 * q:            device bf16 [n_tokens][n_q_heads][128], contiguous.
 * k_cur, v_cur: device bf16 [n_tokens][n_kv_heads][128], contiguous.
 * prefix_rows:  device int32 [n_prefix], physical rows of `pool` (an
 *               out-of-range entry is clamped to num_rows - 1).
 * ws_k, ws_v:   device bf16, each >= n_prefix * n_kv_heads * 128 elements
 *               (ws_capacity_rows >= n_prefix rows); written by step 1, laid
 *               out [n_prefix][n_kv_heads][128]; may be shared by all layers.
 * out:          device bf16 [n_tokens][n_q_heads][128].
 * All bf16 bases 16-byte aligned.  n_tokens >= 1, n_prefix >= 0.
 * Errors: INVALID_ARG, UNSUPPORTED, ALIGNMENT, WORKSPACE (ws too small), HIP.
 */
fp8kv_status fp8kv_prefill_attn(const fp8kv_pool_layer *pool, const uint16_t *q, const uint16_t *k_cur,
                                const uint16_t *v_cur, int32_t n_tokens, int32_t n_q_heads,
                                const int32_t *prefix_rows, int32_t n_prefix, uint16_t *ws_k,
                                uint16_t *ws_v, int64_t ws_capacity_rows, float sm_scale,
                                uint16_t *out, void *stream);

/*
 * fp8kv_prefill_attn_workspace -- step 2 of fp8kv_prefill_attn alone: causal
 * attention of one bf16 chunk over bf16 prefix rows that are already in a
 * workspace (FreeToken PR #853, "What changes": the prefill attends over the
 * BF16 workspace rebuilt once per layer, followed by the BF16 chunk; "Paired
 * end-to-end A/B": the same operator over a BF16 KV pool is the comparison
 * point).  Use it for every further call of a layer whose workspace one
 * fp8kv_prefill_attn call has already rebuilt, or over the rows of a BF16 KV
 * cache.
 *
 * Chunk query i (absolute position n_prefix + i) attends to keys/values
 * [ws rows 0..n_prefix-1 ; chunk rows 0..i] with KV head
 * g = h / (n_q_heads / n_kv_heads) and softmax scale sm_scale; out[i][h] is
 * rounded to bf16 -- step 2 of fp8kv_prefill_attn, bit for bit.
 *
 * q:            device bf16 [n_tokens][n_q_heads][128], contiguous.
 * k_cur, v_cur: device bf16 [n_tokens][n_kv_heads][128], contiguous.
 * ws_k, ws_v:   device bf16 [n_prefix][n_kv_heads][128] (may be NULL when
 *               n_prefix == 0).
 * out:          device bf16 [n_tokens][n_q_heads][128].
 * All bf16 bases 16-byte aligned.  n_tokens >= 1, n_prefix >= 0, n_q_heads a
 * multiple of n_kv_heads with a ratio in {1, 2, 4, 8, 16}.
 * Errors: INVALID_ARG, UNSUPPORTED, ALIGNMENT, WORKSPACE (ws missing), HIP.
 */
fp8kv_status fp8kv_prefill_attn_workspace(const uint16_t *q, const uint16_t *k_cur, const uint16_t *v_cur,
                                          int32_t n_tokens, int32_t n_q_heads, int32_t n_kv_heads,
                                          const uint16_t *ws_k, const uint16_t *ws_v, int32_t n_prefix,
                                          float sm_scale, uint16_t *out, void *stream);

/* Static, human-readable name of a status code. */
const char *fp8kv_status_string(fp8kv_status status);

#ifdef __cplusplus
}
#endif

#endif /* FP8KV_H */
