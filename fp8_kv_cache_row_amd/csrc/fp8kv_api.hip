// fp8kv_api.hip -- the extern "C" boundary of libfp8kv.so (declared in fp8kv.h).
//
// Every check that does not need device memory happens here, before anything
// is enqueued (FreeToken PR #853, "What changes": unsupported combinations are
// rejected up front; PR #897 description: the packed reader requires 16-byte
// aligned bases and row strides).  Kernels live in quantize.hip, decode.hip and
// prefill.hip.
#include <mutex>
#include <string.h>

#include "fp8kv.h"
#include "fp8kv_device.h"

static_assert(FP8KV_MAX_SPLITS == FP8KV_MAX_SPLITS_INTERNAL, "split cap mismatch");
static_assert(FP8KV_MAX_DECODE_GROUPS == FP8KV_MAX_DECODE_GROUPS_INTERNAL, "decode group cap mismatch");
static_assert(FP8KV_CODE_E4M3 == fp8kv::kE4M3 && FP8KV_CODE_INT8 == fp8kv::kInt8, "code format mismatch");

namespace {

using fp8kv::PoolView;

fp8kv_status from_hip(hipError_t e) { return e == hipSuccess ? FP8KV_OK : FP8KV_ERR_HIP; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// A softmax scale must be finite and positive: every kernel takes the running
// maximum of scaled scores, and only a positive finite factor keeps that the
// maximum of the raw scores (zero would also make masked keys 0 * -inf).
// Tested on the bit pattern, independent of floating-point compile flags.
bool valid_softmax_scale(float x) {
  uint32_t u;
  memcpy(&u, &x, sizeof(u));
  return (u & 0x80000000u) == 0u && (u & 0x7f800000u) != 0x7f800000u && u != 0u;
}

bool supported_group(int32_t n_q_heads, int32_t n_kv_heads) {
  if (n_kv_heads <= 0 || n_q_heads <= 0 || n_q_heads % n_kv_heads != 0) return false;
  const int32_t g = n_q_heads / n_kv_heads;
  return g == 1 || g == 2 || g == 4 || g == 8 || g == 16;
}

fp8kv_status check_pool(const fp8kv_pool_layer* p) {
  if (!p || !p->k_codes || !p->v_codes || !p->k_scales || !p->v_scales) return FP8KV_ERR_INVALID_ARG;
  if (p->num_rows <= 0 || p->num_rows > INT32_MAX || p->n_kv_heads <= 0) return FP8KV_ERR_INVALID_ARG;
  if (p->head_dim != FP8KV_HEAD_DIM && p->head_dim != FP8KV_HEAD_DIM_256) return FP8KV_ERR_UNSUPPORTED;
  if (p->code_format != FP8KV_CODE_E4M3 && p->code_format != FP8KV_CODE_INT8) return FP8KV_ERR_UNSUPPORTED;
  if (p->code_row_stride < (int64_t)p->n_kv_heads * p->head_dim) return FP8KV_ERR_INVALID_ARG;
  if (p->scale_row_stride < p->n_kv_heads) return FP8KV_ERR_INVALID_ARG;
  if (!aligned(p->k_codes, 16) || !aligned(p->v_codes, 16) || (p->code_row_stride % 16) != 0)
    return FP8KV_ERR_ALIGNMENT;
  if (!aligned(p->k_scales, 4) || !aligned(p->v_scales, 4)) return FP8KV_ERR_ALIGNMENT;
  return FP8KV_OK;
}

PoolView view_of(const fp8kv_pool_layer* p) {
  const bool line_rows = aligned(p->k_codes, 128) && aligned(p->v_codes, 128) && p->code_row_stride % 128 == 0 &&
                         p->head_dim % 128 == 0;
  return PoolView{p->k_codes, p->v_codes, p->k_scales, p->v_scales, p->code_row_stride, p->scale_row_stride,
                  p->n_kv_heads, p->head_dim, p->num_rows, p->code_format, line_rows};
}

// Per-device facts, queried once: gfx950 or not, and the compute-unit count.
struct DeviceInfo {
  bool known = false;
  bool gfx950 = false;
  int n_cu = 0;
  void* scratch = nullptr;  // device address of `scratch` on this device, once looked up
};
constexpr int kMaxDevices = 64;
std::mutex g_dev_mu;
DeviceInfo g_dev[kMaxDevices];

fp8kv_status current_device(int* n_cu) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FP8KV_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_dev_mu);
  DeviceInfo& info = g_dev[dev];
  if (!info.known) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FP8KV_ERR_HIP;
    info.gfx950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    info.n_cu = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1;
    info.known = true;
  }
  if (!info.gfx950) return FP8KV_ERR_UNSUPPORTED;
  if (n_cu) *n_cu = info.n_cu;
  return FP8KV_OK;
}

int32_t split_cap(int32_t max_splits) {
  return (max_splits > 0 && max_splits < FP8KV_MAX_SPLITS) ? max_splits : FP8KV_MAX_SPLITS;
}

// Split choice: about one stage-1 workgroup per compute unit across the
// batch (a workgroup fills its CU's registers: 8 waves of up to 256 or 4 waves
// of up to 512); a split covers a multiple of 32 keys of the request's key
// span (the window plus the extra query rows with a window, max_seq_len
// otherwise).  When that one round would give splits of more than 2 x 512
// keys (a batch, a long context), splits take 512 keys over several rounds,
// and one-row D = 128 calls switch to the streaming stage-1 shape (three
// 4-wave workgroups per CU).  The split count is padded with empty splits to a
// multiple of 8 (one grid row per XCD) when the workspace cap allows.
// Several query rows put G * n_qrows columns on the MFMA tiles: as many
// 16-column tiles per workgroup as the head dim allows, and more column
// groups beyond that.
#ifndef FP8KV_DECODE_MAX_CHUNK
#define FP8KV_DECODE_MAX_CHUNK 512
#endif
constexpr int64_t kMaxChunkKeys = FP8KV_DECODE_MAX_CHUNK;
#ifndef FP8KV_DECODE_STREAM
#define FP8KV_DECODE_STREAM 1
#endif
constexpr bool kStreamDecode = FP8KV_DECODE_STREAM;

// Column tiles per workgroup and column groups per (request, KV head).
void column_split(int32_t head_dim, int32_t group, int32_t n_qrows, int32_t* col_tiles, int32_t* n_col_groups) {
  *col_tiles = 1;
  *n_col_groups = 1;
  if (n_qrows > 1) {
    const int32_t tiles = (group * n_qrows + 15) / 16;
    const int32_t cap = fp8kv::decode_max_col_tiles(head_dim);
    while (*col_tiles < tiles && *col_tiles < cap) *col_tiles *= 2;
    *n_col_groups = (tiles + *col_tiles - 1) / *col_tiles;
  }
}

fp8kv::DecodeGeometry choose_geometry(int32_t batch, int32_t n_kv_heads, int32_t head_dim, int32_t group,
                                      int32_t n_qrows, int32_t max_seq_len, int32_t window, int32_t max_splits,
                                      int n_cu) {
  int32_t col_tiles, n_col_groups;
  column_split(head_dim, group, n_qrows, &col_tiles, &n_col_groups);
  const int64_t unit = fp8kv::kDecodeTileKeys;
  int64_t span = max_seq_len;
  if (window > 0 && (int64_t)window + n_qrows - 1 < span) span = (int64_t)window + n_qrows - 1;
  const int64_t L = span > 0 ? span : 1;
  const int64_t per = (int64_t)batch * n_kv_heads * n_col_groups;
  const int64_t target = n_cu;
  int64_t want = (target + per - 1) / per;
  if (want < 1) want = 1;
  int64_t ns = want;
  if (ns > split_cap(max_splits)) ns = split_cap(max_splits);
  const int64_t useful = (L + unit - 1) / unit;
  if (ns > useful) ns = useful;
  int64_t chunk = (L + ns - 1) / ns;
  chunk = (chunk + unit - 1) / unit * unit;
  bool stream = false;
  if (kMaxChunkKeys > 0 && chunk > 2 * kMaxChunkKeys) {
    stream = kStreamDecode;
    int64_t ns2 = (L + kMaxChunkKeys - 1) / kMaxChunkKeys;
    if (ns2 > split_cap(max_splits)) ns2 = split_cap(max_splits);
    chunk = (L + ns2 - 1) / ns2;
    chunk = (chunk + unit - 1) / unit * unit;
  }
  ns = (L + chunk - 1) / chunk;
  // Whole rows of 8 splits in the grid (one per XCD); the extra splits start
  // past the span and hold no keys.
  const int64_t ns8 = (ns + 7) / 8 * 8;
  if (ns8 <= split_cap(max_splits)) ns = ns8;
  return fp8kv::DecodeGeometry{(int32_t)ns, (int32_t)chunk, col_tiles, n_col_groups, stream && n_qrows == 1 && window == 0 && head_dim == 128};
}

size_t partial_bytes(int64_t n_queries, int64_t n_q_heads, int64_t head_dim, int64_t split_stride) {
  return fp8kv::kDecodeHeaderBytes + (size_t)(n_queries * n_q_heads * split_stride) * (head_dim + 1) * sizeof(float);
}

fp8kv::DecodeWorkspace workspace_view(void* workspace, int64_t n_queries, int32_t n_q_heads, int32_t head_dim,
                                      int32_t max_splits) {
  const int32_t stride = split_cap(max_splits);
  char* base = static_cast<char*>(workspace);
  float* part_o = reinterpret_cast<float*>(base + fp8kv::kDecodeHeaderBytes);
  float* part_lse = part_o + (size_t)n_queries * n_q_heads * stride * head_dim;
  return fp8kv::DecodeWorkspace{reinterpret_cast<int32_t*>(base), part_o, part_lse, stride};
}

bool valid_head_dim(int32_t d) { return d == FP8KV_HEAD_DIM || d == FP8KV_HEAD_DIM_256; }

// Checks shared by every decode entry point (check_decode_shape), and the
// caller's workspace of the calls that take one (check_decode_workspace).
fp8kv_status check_decode_shape(const fp8kv_pool_layer* pool, const uint16_t* q, int32_t batch, int32_t n_qrows,
                                int32_t n_q_heads, const int32_t* row_table, int64_t table_stride,
                                const int32_t* seq_lens, int32_t max_seq_len, int32_t window, float sm_scale,
                                int32_t max_splits) {
  fp8kv_status st = check_pool(pool);
  if (st != FP8KV_OK) return st;
  if (!q || !row_table || !seq_lens) return FP8KV_ERR_INVALID_ARG;
  if (batch <= 0 || max_seq_len < 0 || max_splits < 0 || table_stride < max_seq_len || table_stride <= 0)
    return FP8KV_ERR_INVALID_ARG;
  if (n_qrows < 1 || n_qrows > FP8KV_MAX_QUERY_ROWS || window < 0) return FP8KV_ERR_INVALID_ARG;
  if ((int64_t)batch * n_qrows > INT32_MAX / 2) return FP8KV_ERR_INVALID_ARG;
  if (n_q_heads <= 0 || n_q_heads % pool->n_kv_heads != 0) return FP8KV_ERR_INVALID_ARG;
  if (!supported_group(n_q_heads, pool->n_kv_heads)) return FP8KV_ERR_UNSUPPORTED;
  {
    int32_t col_tiles, n_col_groups;
    column_split(pool->head_dim, n_q_heads / pool->n_kv_heads, n_qrows, &col_tiles, &n_col_groups);
    if ((int64_t)batch * n_col_groups > FP8KV_MAX_DECODE_GROUPS) return FP8KV_ERR_UNSUPPORTED;
  }
  if (!valid_softmax_scale(sm_scale)) return FP8KV_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(row_table, 4) || !aligned(seq_lens, 4)) return FP8KV_ERR_ALIGNMENT;
  return FP8KV_OK;
}

fp8kv_status check_decode_workspace(const fp8kv_pool_layer* pool, int32_t batch, int32_t n_qrows, int32_t n_q_heads,
                                    int32_t max_splits, const void* workspace, size_t workspace_bytes) {
  if (!workspace ||
      workspace_bytes < partial_bytes((int64_t)batch * n_qrows, n_q_heads, pool->head_dim, split_cap(max_splits)))
    return FP8KV_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return FP8KV_ERR_ALIGNMENT;
  return FP8KV_OK;
}

fp8kv_status check_decode_args(const fp8kv_pool_layer* pool, const uint16_t* q, int32_t batch, int32_t n_qrows,
                               int32_t n_q_heads, const int32_t* row_table, int64_t table_stride,
                               const int32_t* seq_lens, int32_t max_seq_len, int32_t window, float sm_scale,
                               int32_t max_splits, const void* workspace, size_t workspace_bytes) {
  fp8kv_status st = check_decode_shape(pool, q, batch, n_qrows, n_q_heads, row_table, table_stride, seq_lens,
                                       max_seq_len, window, sm_scale, max_splits);
  if (st != FP8KV_OK) return st;
  return check_decode_workspace(pool, batch, n_qrows, n_q_heads, max_splits, workspace, workspace_bytes);
}

// Stage 1 (and the merge unless `app` is given) of one decode call, with the
// geometry and workspace view already fixed.
fp8kv_status launch_decode(const fp8kv_pool_layer* pool, const uint16_t* q, const fp8kv::DecodeShape& shape,
                           float sm_scale, const fp8kv::DecodeGeometry& geo, const fp8kv::DecodeWorkspace& ws,
                           uint16_t* out, const fp8kv::AppendArgs* app, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t n_queries = (int64_t)shape.batch * shape.n_qrows;
  // One query row per request in one workgroup round: stage 1 takes the new
  // token and the plain merge follows; otherwise the appending merge takes it.
  const bool fold = app && fp8kv::decode_stage1_takes_new_token(view_of(pool), shape, geo);
  hipError_t e = fp8kv::launch_decode_stage1(view_of(pool), q, shape, sm_scale, geo, ws, app ? shape.n_qrows : 0,
                                             fold ? app : nullptr, s);
  if (e != hipSuccess) return FP8KV_ERR_HIP;
  if (app && !fold)
    return from_hip(fp8kv::launch_decode_merge_append(view_of(pool), shape.batch, shape.n_q_heads, ws, geo.n_split,
                                                      *app, out, s));
  if (!out) return FP8KV_OK;
  return from_hip(fp8kv::launch_decode_merge(n_queries * shape.n_q_heads, pool->head_dim, ws, geo.n_split, out, s));
}

// A decode call over the caller's workspace (split stride = the split cap).
fp8kv_status run_decode(const fp8kv_pool_layer* pool, const uint16_t* q, int32_t batch, int32_t n_qrows,
                        int32_t n_q_heads, const int32_t* row_table, int64_t table_stride, const int32_t* seq_lens,
                        int32_t max_seq_len, int32_t window, float sm_scale, int32_t max_splits, void* workspace,
                        uint16_t* out, const fp8kv::AppendArgs* app, void* stream) {
  int n_cu = 0;
  fp8kv_status st = current_device(&n_cu);
  if (st != FP8KV_OK) return st;
  const fp8kv::DecodeGeometry geo = choose_geometry(batch, pool->n_kv_heads, pool->head_dim, n_q_heads / pool->n_kv_heads,
                                                    n_qrows, max_seq_len, window, max_splits, n_cu);
  const int64_t n_queries = (int64_t)batch * n_qrows;
  const fp8kv::DecodeWorkspace ws = workspace_view(workspace, n_queries, n_q_heads, pool->head_dim, max_splits);
  const fp8kv::DecodeShape shape{batch, n_qrows, n_q_heads, row_table, table_stride, seq_lens, max_seq_len, window};
  return launch_decode(pool, q, shape, sm_scale, geo, ws, out, app, stream);
}

// The allocation-free decode step keeps its split partials in this array, one
// copy per device, instead of a caller's workspace.  Host code never passes
// the array's name to a kernel (on the host it is only a stand-in for the
// symbol): the device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[FP8KV_NOALLOC_SCRATCH_BYTES];

fp8kv_status device_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FP8KV_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_dev_mu);
  DeviceInfo& info = g_dev[dev];
  if (!info.scratch) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FP8KV_ERR_HIP;
    info.scratch = p;
  }
  *ptr = info.scratch;
  return FP8KV_OK;
}

}  // namespace

extern "C" {

fp8kv_status fp8kv_quantize_rows(const fp8kv_pool_layer* pool, const uint16_t* k, const uint16_t* v,
                                 int64_t src_token_stride, const int32_t* slots, int32_t n_tokens,
                                 void* stream) {
  fp8kv_status st = check_pool(pool);
  if (st != FP8KV_OK) return st;
  if (n_tokens < 0) return FP8KV_ERR_INVALID_ARG;
  if (n_tokens == 0) return FP8KV_OK;
  if (!k || !v || !slots) return FP8KV_ERR_INVALID_ARG;
  if (src_token_stride < (int64_t)pool->n_kv_heads * pool->head_dim) return FP8KV_ERR_INVALID_ARG;
  if ((src_token_stride % 8) != 0 || !aligned(k, 16) || !aligned(v, 16)) return FP8KV_ERR_ALIGNMENT;
  if (!aligned(slots, 4)) return FP8KV_ERR_ALIGNMENT;
  st = current_device(nullptr);
  if (st != FP8KV_OK) return st;
  return from_hip(fp8kv::launch_quantize_rows(view_of(pool), k, v, src_token_stride, slots, n_tokens,
                                              static_cast<hipStream_t>(stream)));
}

size_t fp8kv_decode_workspace_bytes(int32_t n_queries, int32_t n_q_heads, int32_t head_dim, int32_t max_splits) {
  if (n_queries <= 0 || n_q_heads <= 0 || max_splits < 0 || !valid_head_dim(head_dim)) return 0;
  return partial_bytes(n_queries, n_q_heads, head_dim, split_cap(max_splits));
}

fp8kv_status fp8kv_decode_stage1(const fp8kv_pool_layer* pool, const uint16_t* q, int32_t batch,
                                 int32_t n_q_heads, const int32_t* row_table, int64_t table_stride,
                                 const int32_t* seq_lens, int32_t max_seq_len, float sm_scale, int32_t max_splits,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  fp8kv_status st = check_decode_args(pool, q, batch, 1, n_q_heads, row_table, table_stride, seq_lens, max_seq_len, 0,
                                      sm_scale, max_splits, workspace, workspace_bytes);
  if (st != FP8KV_OK) return st;
  return run_decode(pool, q, batch, 1, n_q_heads, row_table, table_stride, seq_lens, max_seq_len, 0, sm_scale,
                    max_splits, workspace, nullptr, nullptr, stream);
}

fp8kv_status fp8kv_decode_stage1_valu(const fp8kv_pool_layer* pool, const uint16_t* q, int32_t batch,
                                      int32_t n_q_heads, const int32_t* row_table, int64_t table_stride,
                                      const int32_t* seq_lens, int32_t max_seq_len, float sm_scale,
                                      int32_t max_splits, void* workspace, size_t workspace_bytes, void* stream) {
  fp8kv_status st = check_decode_args(pool, q, batch, 1, n_q_heads, row_table, table_stride, seq_lens, max_seq_len, 0,
                                      sm_scale, max_splits, workspace, workspace_bytes);
  if (st != FP8KV_OK) return st;
  if (pool->head_dim != FP8KV_HEAD_DIM || pool->code_format != FP8KV_CODE_E4M3) return FP8KV_ERR_UNSUPPORTED;
  int n_cu = 0;
  st = current_device(&n_cu);
  if (st != FP8KV_OK) return st;
  const fp8kv::DecodeGeometry geo = choose_geometry(batch, pool->n_kv_heads, pool->head_dim, n_q_heads / pool->n_kv_heads,
                                                    1, max_seq_len, 0, max_splits, n_cu);
  const fp8kv::DecodeWorkspace ws = workspace_view(workspace, batch, n_q_heads, pool->head_dim, max_splits);
  const fp8kv::DecodeShape shape{batch, 1, n_q_heads, row_table, table_stride, seq_lens, max_seq_len, 0};
  return from_hip(fp8kv::launch_decode_stage1_valu(view_of(pool), q, shape, sm_scale, geo, ws,
                                                   static_cast<hipStream_t>(stream)));
}

fp8kv_status fp8kv_decode_merge(int32_t n_queries, int32_t n_q_heads, int32_t head_dim, int32_t max_splits,
                                const void* workspace, size_t workspace_bytes, uint16_t* out, void* stream) {
  if (n_queries <= 0 || n_q_heads <= 0 || max_splits < 0 || !out) return FP8KV_ERR_INVALID_ARG;
  if (!valid_head_dim(head_dim)) return FP8KV_ERR_UNSUPPORTED;
  if ((int64_t)n_queries * n_q_heads > INT32_MAX) return FP8KV_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < partial_bytes(n_queries, n_q_heads, head_dim, split_cap(max_splits)))
    return FP8KV_ERR_WORKSPACE;
  if (!aligned(workspace, 256) || !aligned(out, 16)) return FP8KV_ERR_ALIGNMENT;
  fp8kv_status st = current_device(nullptr);
  if (st != FP8KV_OK) return st;
  const fp8kv::DecodeWorkspace ws =
      workspace_view(const_cast<void*>(workspace), n_queries, n_q_heads, head_dim, max_splits);
  return from_hip(fp8kv::launch_decode_merge((int64_t)n_queries * n_q_heads, head_dim, ws, -1, out,
                                             static_cast<hipStream_t>(stream)));
}

fp8kv_status fp8kv_decode_attn(const fp8kv_pool_layer* pool, const uint16_t* q, int32_t batch,
                               int32_t n_q_heads, const int32_t* row_table, int64_t table_stride,
                               const int32_t* seq_lens, int32_t max_seq_len, float sm_scale,
                               int32_t max_splits, void* workspace, size_t workspace_bytes, uint16_t* out,
                               void* stream) {
  return fp8kv_decode_attn_rows(pool, q, batch, 1, n_q_heads, row_table, table_stride, seq_lens, max_seq_len, 0,
                                sm_scale, max_splits, workspace, workspace_bytes, out, stream);
}

fp8kv_status fp8kv_decode_attn_rows(const fp8kv_pool_layer* pool, const uint16_t* q, int32_t batch, int32_t n_qrows,
                                    int32_t n_q_heads, const int32_t* row_table, int64_t table_stride,
                                    const int32_t* seq_lens, int32_t max_seq_len, int32_t window, float sm_scale,
                                    int32_t max_splits, void* workspace, size_t workspace_bytes, uint16_t* out,
                                    void* stream) {
  fp8kv_status st = check_decode_args(pool, q, batch, n_qrows, n_q_heads, row_table, table_stride, seq_lens,
                                      max_seq_len, window, sm_scale, max_splits, workspace, workspace_bytes);
  if (st != FP8KV_OK) return st;
  if (!out) return FP8KV_ERR_INVALID_ARG;
  if (!aligned(out, 16)) return FP8KV_ERR_ALIGNMENT;
  return run_decode(pool, q, batch, n_qrows, n_q_heads, row_table, table_stride, seq_lens, max_seq_len, window,
                    sm_scale, max_splits, workspace, out, nullptr, stream);
}

fp8kv_status fp8kv_decode_attn_append_window(const fp8kv_pool_layer* pool, const uint16_t* q, int32_t batch,
                                             int32_t n_q_heads, const uint16_t* k_new, const uint16_t* v_new,
                                             int64_t new_token_stride, const int32_t* new_slots,
                                             const int32_t* row_table, int64_t table_stride,
                                             const int32_t* seq_lens, int32_t max_seq_len, int32_t window,
                                             float sm_scale, int32_t max_splits, void* workspace,
                                             size_t workspace_bytes, uint16_t* out, void* stream) {
  fp8kv_status st = check_decode_args(pool, q, batch, 1, n_q_heads, row_table, table_stride, seq_lens, max_seq_len,
                                      window, sm_scale, max_splits, workspace, workspace_bytes);
  if (st != FP8KV_OK) return st;
  if (!out || !k_new || !v_new || !new_slots || max_seq_len < 1) return FP8KV_ERR_INVALID_ARG;
  if (!aligned(new_slots, 4)) return FP8KV_ERR_ALIGNMENT;
  if (new_token_stride < (int64_t)pool->n_kv_heads * pool->head_dim) return FP8KV_ERR_INVALID_ARG;
  if (!aligned(out, 16) || !aligned(k_new, 16) || !aligned(v_new, 16) || (new_token_stride % 8) != 0)
    return FP8KV_ERR_ALIGNMENT;
  const fp8kv::AppendArgs app{q, k_new, v_new, new_token_stride, new_slots, sm_scale, 1, window};
  // Stage 1 covers the window's cached positions [p - window + 1, p); the new
  // token at p is always inside the window, and the merge adds it.
  return run_decode(pool, q, batch, 1, n_q_heads, row_table, table_stride, seq_lens, max_seq_len, window, sm_scale,
                    max_splits, workspace, out, &app, stream);
}

fp8kv_status fp8kv_decode_attn_rows_append(const fp8kv_pool_layer* pool, const uint16_t* q, int32_t batch,
                                           int32_t n_qrows, int32_t n_q_heads, const uint16_t* k_new,
                                           const uint16_t* v_new, int64_t new_token_stride,
                                           const int32_t* new_slots, const int32_t* row_table, int64_t table_stride,
                                           const int32_t* seq_lens, int32_t max_seq_len, int32_t window,
                                           float sm_scale, int32_t max_splits, void* workspace,
                                           size_t workspace_bytes, uint16_t* out, void* stream) {
  fp8kv_status st = check_decode_args(pool, q, batch, n_qrows, n_q_heads, row_table, table_stride, seq_lens,
                                      max_seq_len, window, sm_scale, max_splits, workspace, workspace_bytes);
  if (st != FP8KV_OK) return st;
  if (!out || !k_new || !v_new || !new_slots || max_seq_len < n_qrows) return FP8KV_ERR_INVALID_ARG;
  if (!aligned(new_slots, 4)) return FP8KV_ERR_ALIGNMENT;
  if (new_token_stride < (int64_t)pool->n_kv_heads * pool->head_dim) return FP8KV_ERR_INVALID_ARG;
  if (!aligned(out, 16) || !aligned(k_new, 16) || !aligned(v_new, 16) || (new_token_stride % 8) != 0)
    return FP8KV_ERR_ALIGNMENT;
  const fp8kv::AppendArgs app{q, k_new, v_new, new_token_stride, new_slots, sm_scale, n_qrows, window};
  // Stage 1 covers the cached positions below the request's n_qrows new
  // tokens; the merge of query row i adds the new tokens j <= i in its window.
  return run_decode(pool, q, batch, n_qrows, n_q_heads, row_table, table_stride, seq_lens, max_seq_len, window,
                    sm_scale, max_splits, workspace, out, &app, stream);
}

fp8kv_status fp8kv_decode_attn_append(const fp8kv_pool_layer* pool, const uint16_t* q, int32_t batch,
                                      int32_t n_q_heads, const uint16_t* k_new, const uint16_t* v_new,
                                      int64_t new_token_stride, const int32_t* new_slots,
                                      const int32_t* row_table, int64_t table_stride,
                                      const int32_t* seq_lens, int32_t max_seq_len, float sm_scale,
                                      int32_t max_splits, void* workspace, size_t workspace_bytes, uint16_t* out,
                                      void* stream) {
  return fp8kv_decode_attn_append_window(pool, q, batch, n_q_heads, k_new, v_new, new_token_stride, new_slots,
                                         row_table, table_stride, seq_lens, max_seq_len, 0, sm_scale, max_splits,
                                         workspace, workspace_bytes, out, stream);
}

fp8kv_status fp8kv_decode_attn_append_noalloc(const fp8kv_pool_layer* pool, const uint16_t* q, int32_t batch,
                                              int32_t n_q_heads, const uint16_t* k_new, const uint16_t* v_new,
                                              int64_t new_token_stride, const int32_t* new_slots,
                                              const int32_t* row_table, int64_t table_stride,
                                              const int32_t* seq_lens, int32_t max_seq_len, float sm_scale,
                                              int32_t max_splits, uint16_t* out, void* stream) {
  fp8kv_status st = check_decode_shape(pool, q, batch, 1, n_q_heads, row_table, table_stride, seq_lens, max_seq_len,
                                       0, sm_scale, max_splits);
  if (st != FP8KV_OK) return st;
  if (!out || !k_new || !v_new || !new_slots || max_seq_len < 1) return FP8KV_ERR_INVALID_ARG;
  if (!aligned(new_slots, 4)) return FP8KV_ERR_ALIGNMENT;
  if (new_token_stride < (int64_t)pool->n_kv_heads * pool->head_dim) return FP8KV_ERR_INVALID_ARG;
  if (!aligned(out, 16) || !aligned(k_new, 16) || !aligned(v_new, 16) || (new_token_stride % 8) != 0)
    return FP8KV_ERR_ALIGNMENT;
  int n_cu = 0;
  st = current_device(&n_cu);
  if (st != FP8KV_OK) return st;
  // The partials are laid out with a split stride of exactly the split count
  // this launch uses, so the array holds as many (request, head) rows as fit.
  const fp8kv::DecodeGeometry geo =
      choose_geometry(batch, pool->n_kv_heads, pool->head_dim, n_q_heads / pool->n_kv_heads, 1, max_seq_len, 0,
                      max_splits, n_cu);
  const size_t need = partial_bytes(batch, n_q_heads, pool->head_dim, geo.n_split);
  if (need > (size_t)FP8KV_NOALLOC_SCRATCH_BYTES) return FP8KV_ERR_WORKSPACE;
  void* base = nullptr;
  st = device_scratch(&base);
  if (st != FP8KV_OK) return st;
  char* b = static_cast<char*>(base);
  float* part_o = reinterpret_cast<float*>(b + fp8kv::kDecodeHeaderBytes);
  const fp8kv::DecodeWorkspace ws{reinterpret_cast<int32_t*>(b), part_o,
                                  part_o + (size_t)batch * n_q_heads * geo.n_split * pool->head_dim, geo.n_split};
  const fp8kv::DecodeShape shape{batch, 1, n_q_heads, row_table, table_stride, seq_lens, max_seq_len, 0};
  const fp8kv::AppendArgs app{q, k_new, v_new, new_token_stride, new_slots, sm_scale, 1, 0};
  return launch_decode(pool, q, shape, sm_scale, geo, ws, out, &app, stream);
}

fp8kv_status fp8kv_prefill_attn(const fp8kv_pool_layer* pool, const uint16_t* q, const uint16_t* k_cur,
                                const uint16_t* v_cur, int32_t n_tokens, int32_t n_q_heads,
                                const int32_t* prefix_rows, int32_t n_prefix, uint16_t* ws_k, uint16_t* ws_v,
                                int64_t ws_capacity_rows, float sm_scale, uint16_t* out, void* stream) {
  fp8kv_status st = check_pool(pool);
  if (st != FP8KV_OK) return st;
  if (pool->head_dim != FP8KV_HEAD_DIM) return FP8KV_ERR_UNSUPPORTED;
  if (!q || !k_cur || !v_cur || !out) return FP8KV_ERR_INVALID_ARG;
  if (n_tokens <= 0 || n_prefix < 0) return FP8KV_ERR_INVALID_ARG;
  if (n_q_heads <= 0 || n_q_heads % pool->n_kv_heads != 0) return FP8KV_ERR_INVALID_ARG;
  if (!supported_group(n_q_heads, pool->n_kv_heads)) return FP8KV_ERR_UNSUPPORTED;
  if (!valid_softmax_scale(sm_scale)) return FP8KV_ERR_INVALID_ARG;
  if (n_prefix > 0) {
    if (!prefix_rows) return FP8KV_ERR_INVALID_ARG;
    if (!ws_k || !ws_v || ws_capacity_rows < n_prefix) return FP8KV_ERR_WORKSPACE;
    if (!aligned(ws_k, 16) || !aligned(ws_v, 16) || !aligned(prefix_rows, 4)) return FP8KV_ERR_ALIGNMENT;
  }
  if (!aligned(q, 16) || !aligned(k_cur, 16) || !aligned(v_cur, 16) || !aligned(out, 16))
    return FP8KV_ERR_ALIGNMENT;
  st = current_device(nullptr);
  if (st != FP8KV_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (n_prefix > 0) {
    hipError_t e = fp8kv::launch_reconstruct(view_of(pool), prefix_rows, n_prefix, ws_k, ws_v, s);
    if (e != hipSuccess) return FP8KV_ERR_HIP;
  }
  return from_hip(fp8kv::launch_prefill_attention(q, ws_k, ws_v, k_cur, v_cur, n_prefix, n_tokens, n_q_heads,
                                                  pool->n_kv_heads, sm_scale, out, s));
}

fp8kv_status fp8kv_prefill_attn_workspace(const uint16_t* q, const uint16_t* k_cur, const uint16_t* v_cur,
                                          int32_t n_tokens, int32_t n_q_heads, int32_t n_kv_heads,
                                          const uint16_t* ws_k, const uint16_t* ws_v, int32_t n_prefix, float sm_scale,
                                          uint16_t* out, void* stream) {
  if (!q || !k_cur || !v_cur || !out) return FP8KV_ERR_INVALID_ARG;
  if (n_tokens <= 0 || n_prefix < 0 || n_kv_heads <= 0) return FP8KV_ERR_INVALID_ARG;
  if (n_q_heads <= 0 || n_q_heads % n_kv_heads != 0) return FP8KV_ERR_INVALID_ARG;
  if (!supported_group(n_q_heads, n_kv_heads)) return FP8KV_ERR_UNSUPPORTED;
  if (!valid_softmax_scale(sm_scale)) return FP8KV_ERR_INVALID_ARG;
  if (n_prefix > 0 && (!ws_k || !ws_v)) return FP8KV_ERR_WORKSPACE;
  if (n_prefix > 0 && (!aligned(ws_k, 16) || !aligned(ws_v, 16))) return FP8KV_ERR_ALIGNMENT;
  if (!aligned(q, 16) || !aligned(k_cur, 16) || !aligned(v_cur, 16) || !aligned(out, 16))
    return FP8KV_ERR_ALIGNMENT;
  fp8kv_status st = current_device(nullptr);
  if (st != FP8KV_OK) return st;
  return from_hip(fp8kv::launch_prefill_attention(q, ws_k, ws_v, k_cur, v_cur, n_prefix, n_tokens, n_q_heads,
                                                  n_kv_heads, sm_scale, out, static_cast<hipStream_t>(stream)));
}

const char* fp8kv_status_string(fp8kv_status status) {
  switch (status) {
    case FP8KV_OK: return "FP8KV_OK";
    case FP8KV_ERR_INVALID_ARG: return "FP8KV_ERR_INVALID_ARG: null pointer or invalid size";
    case FP8KV_ERR_UNSUPPORTED: return "FP8KV_ERR_UNSUPPORTED: head_dim, GQA ratio or device not supported";
    case FP8KV_ERR_ALIGNMENT: return "FP8KV_ERR_ALIGNMENT: pointer or stride breaks the alignment contract";
    case FP8KV_ERR_WORKSPACE: return "FP8KV_ERR_WORKSPACE: workspace missing or too small";
    case FP8KV_ERR_HIP: return "FP8KV_ERR_HIP: HIP runtime error";
  }
  return "FP8KV_ERR_UNKNOWN";
}

}  // extern "C"
