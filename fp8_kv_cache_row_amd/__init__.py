"""FP8 (OCP E4M3FN) per-row KV cache and GQA decode/prefill attention for MI355X.

The compute lives in libfp8kv.so (hand-written HIP for gfx950, C ABI declared
in include/fp8kv.h); `binding` is a ctypes layer with the same call names and
`workloads` builds seeded synthetic inputs.  Importing this package does not
load the library; the first call does, and fails loudly if it is not built.
"""
from .binding import (Fp8KvError, Fp8KvPool, PoolLayer, decode_workspace, fp8kv_decode_attn,
                      fp8kv_decode_attn_append, fp8kv_decode_attn_rows, fp8kv_decode_attn_rows_append,
                      fp8kv_decode_merge, fp8kv_decode_stage1,
                      fp8kv_decode_workspace_bytes, fp8kv_prefill_attn, fp8kv_prefill_attn_workspace,
                      fp8kv_quantize_rows, load, status_string)

__all__ = ["Fp8KvError", "Fp8KvPool", "PoolLayer", "decode_workspace", "fp8kv_decode_attn",
           "fp8kv_decode_attn_append", "fp8kv_decode_attn_rows", "fp8kv_decode_attn_rows_append",
           "fp8kv_decode_merge", "fp8kv_decode_stage1",
           "fp8kv_decode_workspace_bytes", "fp8kv_prefill_attn", "fp8kv_prefill_attn_workspace",
           "fp8kv_quantize_rows", "load",
           "status_string"]
