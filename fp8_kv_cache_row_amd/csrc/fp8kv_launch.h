// fp8kv_launch.h -- internal launch entry points of the gfx950 kernels.
// The C ABI (fp8kv_api.hip) validates every argument before calling these.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8kv {

// Row indices read from device memory (table entries, slots, prefix rows) are
// clamped to [0, num_rows) by every kernel, so no table content can make a
// kernel address memory outside the pool.
struct PoolView {
  uint8_t* k_codes;
  uint8_t* v_codes;
  float* k_scales;
  float* v_scales;
  int64_t code_row_stride;   // bytes
  int64_t scale_row_stride;  // floats
  int32_t n_kv_heads;
  int32_t head_dim;  // 128 or 256
  int64_t num_rows;
  int32_t format;    // CodeFormat: 0 E4M3FN, 1 INT8
  // Every KV head's K and V code rows start on a 128-byte line and fill whole
  // lines (bases and row stride multiples of 128 bytes): no two KV heads read
  // the same line, so the decode kernels stream the codes with non-temporal
  // loads.
  bool line_rows;
};

// Decode launch geometry: each workgroup covers `chunk` consecutive keys of
// one (request, KV head, column group); `n_split` workgroups per (request, KV
// head, column group).  A column is one (query row, query head) pair of a KV
// head; a workgroup holds `col_tiles` tiles of 16 columns, and `n_col_groups`
// workgroups cover all G * n_qrows columns (one row per request: 1 and 1).
struct DecodeGeometry {
  int32_t n_split;
  int32_t chunk;  // multiple of kDecodeTileKeys
  int32_t col_tiles;
  int32_t n_col_groups;
  // Several workgroup rounds per compute unit: 4-wave workgroups of at most
  // 168 registers, so three share a compute unit and one's loads cover the
  // others' start-up and epilogue.
  bool stream;
};

// The decode problem: q [batch][n_qrows][n_q_heads][head_dim]; query row i of
// request b sits at position seq_lens[b] - n_qrows + i and sees positions
// [max(0, p - window + 1), p] (window <= 0: [0, p]).
struct DecodeShape {
  int32_t batch;
  int32_t n_qrows;
  int32_t n_q_heads;
  const int32_t* row_table;
  int64_t table_stride;
  const int32_t* seq_lens;
  int32_t max_seq_len;
  int32_t window;
};

#ifndef FP8KV_DECODE_WAVES
#define FP8KV_DECODE_WAVES 8
#endif
#ifndef FP8KV_DECODE_TILES_PER_WAVE
#define FP8KV_DECODE_TILES_PER_WAVE 2
#endif
// Must equal FP8KV_MAX_SPLITS of the public header (checked in the C ABI).
#define FP8KV_MAX_SPLITS_INTERNAL 256
// Requests (times column groups) per decode launch: they share one grid dimension.
#define FP8KV_MAX_DECODE_GROUPS_INTERNAL 65535

constexpr int kDecodeWaves = FP8KV_DECODE_WAVES;                 // waves per stage-1 workgroup (narrow shapes)
constexpr int kDecodeTileKeys = 32;                              // keys per wave per MFMA step
constexpr int kDecodeTilesPerWave = FP8KV_DECODE_TILES_PER_WAVE;  // steps in flight per wave (D = 128, one tile)

hipError_t launch_quantize_rows(const PoolView& pool, const uint16_t* k, const uint16_t* v,
                                int64_t src_token_stride, const int32_t* slots, int32_t n_tokens,
                                hipStream_t stream);

hipError_t launch_reconstruct(const PoolView& pool, const int32_t* prefix_rows, int32_t n_prefix,
                              uint16_t* ws_k, uint16_t* ws_v, hipStream_t stream);

// Split-K partials in the caller's workspace: a 256-byte header whose first
// int32 is the split count of the last stage-1 launch, then
// o[B * n_qrows][Hq][split_stride][head_dim] and lse[B * n_qrows][Hq][split_stride]
// (fp32, log2 units).
struct DecodeWorkspace {
  int32_t* header;
  float* part_o;
  float* part_lse;
  int32_t split_stride;
};
constexpr size_t kDecodeHeaderBytes = 256;

// Column tiles one stage-1 workgroup can hold at this head dim.
int32_t decode_max_col_tiles(int32_t head_dim);

struct AppendArgs;

// key_trim = n_qrows (an appending call) leaves each request's last n_qrows
// keys, its new tokens, out of the cached keys.  Those are then taken by the
// appending merge below, or, with `fold` (one query row per request, where
// decode_stage1_takes_new_token holds), by stage 1 itself: split 0's
// workgroup of each (request, KV head) quantizes the new token into its pool
// row and folds it into that split's partial, and the plain merge follows.
bool decode_stage1_takes_new_token(const PoolView& pool, const DecodeShape& shape, const DecodeGeometry& geo);
hipError_t launch_decode_stage1(const PoolView& pool, const uint16_t* q, const DecodeShape& shape, float sm_scale,
                                const DecodeGeometry& geo, const DecodeWorkspace& ws, int32_t key_trim,
                                const AppendArgs* fold, hipStream_t stream);

// The VALU-only stage 1 (no matrix instructions), same grid and partials:
// head dim 128, E4M3 codes, one query row, no window.
hipError_t launch_decode_stage1_valu(const PoolView& pool, const uint16_t* q, const DecodeShape& shape,
                                     float sm_scale, const DecodeGeometry& geo, const DecodeWorkspace& ws,
                                     hipStream_t stream);

// n_split < 0: take the split count the preceding stage 1 wrote into the
// header.  n_rows_heads = batch * n_qrows * n_q_heads output vectors.
hipError_t launch_decode_merge(int64_t n_rows_heads, int32_t head_dim, const DecodeWorkspace& ws, int32_t n_split,
                               uint16_t* out, hipStream_t stream);

// The new token of each request: bf16 K/V rows [B][token_stride] (head g at
// g * head_dim), quantized into pool row new_slots[b] and folded in as one
// more key, by stage 1 (see above) or by the merge as one more single-key
// partial.
struct AppendArgs {
  const uint16_t* q;
  const uint16_t* k_new;
  const uint16_t* v_new;
  int64_t new_token_stride;  // elements
  const int32_t* new_slots;  // [batch][n_qrows]
  float sm_scale;
  int32_t n_qrows;  // new tokens per request, the request's last n_qrows positions
  int32_t window;   // sliding key window (0: none)
};
hipError_t launch_decode_merge_append(const PoolView& pool, int32_t batch, int32_t n_q_heads, const DecodeWorkspace& ws,
                                      int32_t n_split, const AppendArgs& app, uint16_t* out, hipStream_t stream);

hipError_t launch_prefill_attention(const uint16_t* q, const uint16_t* ws_k, const uint16_t* ws_v,
                                    const uint16_t* k_cur, const uint16_t* v_cur, int32_t n_prefix,
                                    int32_t n_tokens, int32_t n_q_heads, int32_t n_kv_heads,
                                    float sm_scale, uint16_t* out, hipStream_t stream);

}  // namespace fp8kv
