/* abi_from_c.c -- the C ABI used from plain C99 with no GPU: the header
 * compiles as C, the library links, and host-side validation answers before
 * any device work (every call below is rejected on the host). */
#include <stdio.h>
#include <string.h>

#include "fp8kv.h"

static int fails = 0;

static void expect(const char *what, fp8kv_status got, fp8kv_status want) {
    if (got != want) {
        printf("FAIL %s: got %d (%s), want %d\n", what, (int)got, fp8kv_status_string(got), (int)want);
        ++fails;
    }
}

int main(void) {
    static unsigned char fake[4096] __attribute__((aligned(256)));  /* never dereferenced */
    fp8kv_pool_layer pool;
    memset(&pool, 0, sizeof pool);
    pool.k_codes = fake;
    pool.v_codes = fake;
    pool.k_scales = (float *)fake;
    pool.v_scales = (float *)fake;
    pool.num_rows = 16;
    pool.n_kv_heads = 4;
    pool.head_dim = FP8KV_HEAD_DIM;
    pool.code_row_stride = 4 * FP8KV_HEAD_DIM;
    pool.scale_row_stride = 4;
    pool.code_format = FP8KV_CODE_E4M3;

    if (sizeof(fp8kv_pool_layer) != 72) {
        printf("FAIL sizeof(fp8kv_pool_layer) = %zu\n", sizeof(fp8kv_pool_layer));
        ++fails;
    }
    if (strncmp(fp8kv_status_string(FP8KV_ERR_ALIGNMENT), "FP8KV_ERR_ALIGNMENT", 19) != 0) ++fails;
    if (fp8kv_decode_workspace_bytes(1, 32, FP8KV_HEAD_DIM, 64) != 256 + (size_t)32 * 64 * 129 * 4) ++fails;
    if (fp8kv_decode_workspace_bytes(1, 32, 64, 64) != 0) ++fails;

    expect("quantize: null pool", fp8kv_quantize_rows(NULL, NULL, NULL, 0, NULL, 1, NULL), FP8KV_ERR_INVALID_ARG);
    pool.head_dim = 96;
    expect("quantize: head_dim 96", fp8kv_quantize_rows(&pool, (uint16_t *)fake, (uint16_t *)fake, 512,
                                                        (int32_t *)fake, 1, NULL), FP8KV_ERR_UNSUPPORTED);
    pool.head_dim = FP8KV_HEAD_DIM;
    pool.code_format = 7;
    expect("quantize: code format 7", fp8kv_quantize_rows(&pool, (uint16_t *)fake, (uint16_t *)fake, 512,
                                                          (int32_t *)fake, 1, NULL), FP8KV_ERR_UNSUPPORTED);
    pool.code_format = FP8KV_CODE_INT8;
    expect("quantize: zero tokens", fp8kv_quantize_rows(&pool, NULL, NULL, 0, NULL, 0, NULL), FP8KV_OK);
    expect("decode: G = 3", fp8kv_decode_attn(&pool, (uint16_t *)fake, 1, 12, (int32_t *)fake, 64, (int32_t *)fake,
                                              64, 0.088f, 0, fake, sizeof fake, (uint16_t *)fake, NULL),
           FP8KV_ERR_UNSUPPORTED);
    expect("decode: workspace", fp8kv_decode_attn(&pool, (uint16_t *)fake, 1, 32, (int32_t *)fake, 64,
                                                  (int32_t *)fake, 64, 0.088f, 0, fake, 100, (uint16_t *)fake, NULL),
           FP8KV_ERR_WORKSPACE);
    expect("rows: 9 query rows", fp8kv_decode_attn_rows(&pool, (uint16_t *)fake, 1, 9, 32, (int32_t *)fake, 64,
                                                        (int32_t *)fake, 64, 0, 0.088f, 0, fake, sizeof fake,
                                                        (uint16_t *)fake, NULL), FP8KV_ERR_INVALID_ARG);
    expect("merge: misaligned out", fp8kv_decode_merge(1, 4, FP8KV_HEAD_DIM, 1, fake, sizeof fake,
                                                       (uint16_t *)(fake + 2), NULL), FP8KV_ERR_ALIGNMENT);
    expect("prefill: null q", fp8kv_prefill_attn(&pool, NULL, (uint16_t *)fake, (uint16_t *)fake, 4, 32, NULL, 0,
                                                 NULL, NULL, 0, 0.088f, (uint16_t *)fake, NULL),
           FP8KV_ERR_INVALID_ARG);
    printf("%s\n", fails ? "abi_from_c: FAILED" : "abi_from_c: ok");
    return fails ? 1 : 0;
}
