// quantize.hip -- quantize-on-write of K/V rows and the prefill reconstruction.
//
// FreeToken PR #853 "opt-in FP8 KV cache", "What changes": each physical K/V
// row stores E4M3 codes as bytes plus its own FP32 scale; the prefill path
// rebuilds historical FP8 rows once per layer into a shared BF16 workspace.
// "Follow-up model/workload search": the FP8 path quantizes every new K/V row.
//
// Both kernels give one row of D elements to D/8 lanes (8 elements, 16 bytes
// of bf16 or 8 bytes of codes per lane), so a wave handles 64*8/D rows with
// fully coalesced row accesses and the row reduction stays inside 16 or 32
// lanes.  Quantize covers head dims 128 and 256; the reconstruction serves
// the D = 128 prefill.
#include "fp8kv_device.h"

namespace fp8kv {

namespace {

constexpr int kBlock = 256;

// Rows are enumerated as ((token * 2 + kv) * n_kv_heads + head), kv 0 = K, 1 = V.
// F is the code format (E4M3FN, or the symmetric INT8 counterpart).
template <int D, int F>
__global__ __launch_bounds__(kBlock) void quantize_rows_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int64_t src_token_stride,
    const int32_t* __restrict__ slots, int64_t n_rows, int32_t n_kv_heads, uint8_t* __restrict__ k_codes,
    uint8_t* __restrict__ v_codes, float* __restrict__ k_scales, float* __restrict__ v_scales,
    int64_t code_row_stride, int64_t scale_row_stride, uint32_t max_row) {
  constexpr int kLanesPerRow = D / 8;
  constexpr int kRowsPerBlock = kBlock / kLanesPerRow;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x / kLanesPerRow);
  const int sub = threadIdx.x % kLanesPerRow;
  if (row >= n_rows) return;  // whole 16-lane groups leave together
  const int32_t g = (int32_t)(row % n_kv_heads);
  const int64_t tk = row / n_kv_heads;
  const int kv = (int)(tk & 1);
  const int64_t t = tk >> 1;

  const uint16_t* src = (kv ? v : k) + t * src_token_stride + (int64_t)g * D + sub * 8;
  const uint4 raw = *reinterpret_cast<const uint4*>(src);
  float x[8] = {bf16lo_to_f32(raw.x), bf16hi_to_f32(raw.x), bf16lo_to_f32(raw.y), bf16hi_to_f32(raw.y),
                bf16lo_to_f32(raw.z), bf16hi_to_f32(raw.z), bf16lo_to_f32(raw.w), bf16hi_to_f32(raw.w)};

  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
  for (int off = kLanesPerRow / 2; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kLanesPerRow));

  using C = Codec<F>;
  const float s = C::scale(amax);
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = C::prescale(x[i], amax, s);
  uint32_t lo = C::template pack2<false>(y[0], y[1], 0u);
  lo = C::template pack2<true>(y[2], y[3], lo);
  uint32_t hi = C::template pack2<false>(y[4], y[5], 0u);
  hi = C::template pack2<true>(y[6], y[7], hi);

  const int64_t slot = min((uint32_t)slots[t], max_row);  // out-of-range slots are clamped, never followed
  uint8_t* dst = (kv ? v_codes : k_codes) + slot * code_row_stride + (int64_t)g * D + sub * 8;
  *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
  if (sub == 0) (kv ? v_scales : k_scales)[slot * scale_row_stride + g] = s;
}

// Rows enumerated as ((j * 2 + kv) * n_kv_heads + head) for prefix position j.
// ws[j][head][d] = bf16_rne(fl32(decode(code) * scale)).
constexpr int kLanesPerRow = kHeadDim / 8;
constexpr int kRowsPerBlock = kBlock / kLanesPerRow;
template <int F>
__global__ __launch_bounds__(kBlock) void reconstruct_kernel(
    const uint8_t* __restrict__ k_codes, const uint8_t* __restrict__ v_codes,
    const float* __restrict__ k_scales, const float* __restrict__ v_scales, int64_t code_row_stride,
    int64_t scale_row_stride, const int32_t* __restrict__ prefix_rows, int64_t n_rows, int32_t n_kv_heads,
    uint32_t max_row, uint16_t* __restrict__ ws_k, uint16_t* __restrict__ ws_v) {
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x / kLanesPerRow);
  const int sub = threadIdx.x % kLanesPerRow;
  if (row >= n_rows) return;
  const int32_t g = (int32_t)(row % n_kv_heads);
  const int64_t jk = row / n_kv_heads;
  const int kv = (int)(jk & 1);
  const int64_t j = jk >> 1;
  const int64_t prow = min((uint32_t)prefix_rows[j], max_row);

  const uint8_t* src = (kv ? v_codes : k_codes) + prow * code_row_stride + (int64_t)g * kHeadDim + sub * 8;
  const uint2 c = *reinterpret_cast<const uint2*>(src);
  const float s = (kv ? v_scales : k_scales)[prow * scale_row_stride + g];
  float f[8];
  Codec<F>::widen4(c.x, f);
  Codec<F>::widen4(c.y, f + 4);
  uint4 o;
  o.x = f32x2_to_bf16x2(f[0] * s, f[1] * s);
  o.y = f32x2_to_bf16x2(f[2] * s, f[3] * s);
  o.z = f32x2_to_bf16x2(f[4] * s, f[5] * s);
  o.w = f32x2_to_bf16x2(f[6] * s, f[7] * s);
  uint16_t* dst = (kv ? ws_v : ws_k) + (j * n_kv_heads + g) * kHeadDim + sub * 8;
  *reinterpret_cast<uint4*>(dst) = o;
}

template <int D, int F>
void launch_quantize_df(const PoolView& pool, const uint16_t* k, const uint16_t* v, int64_t src_token_stride,
                        const int32_t* slots, int64_t n_rows, hipStream_t stream) {
  constexpr int rows_per_block = kBlock / (D / 8);
  const int64_t blocks = (n_rows + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL((quantize_rows_kernel<D, F>), dim3((unsigned)blocks), dim3(kBlock), 0, stream, k, v,
                     src_token_stride, slots, n_rows, pool.n_kv_heads, pool.k_codes, pool.v_codes, pool.k_scales,
                     pool.v_scales, pool.code_row_stride, pool.scale_row_stride, (uint32_t)(pool.num_rows - 1));
}

}  // namespace

hipError_t launch_quantize_rows(const PoolView& pool, const uint16_t* k, const uint16_t* v,
                                int64_t src_token_stride, const int32_t* slots, int32_t n_tokens,
                                hipStream_t stream) {
  const int64_t n_rows = (int64_t)n_tokens * 2 * pool.n_kv_heads;
  if (n_rows == 0) return hipSuccess;
  const bool i8 = pool.format == kInt8;
  if (pool.head_dim == 128)
    i8 ? launch_quantize_df<128, kInt8>(pool, k, v, src_token_stride, slots, n_rows, stream)
       : launch_quantize_df<128, kE4M3>(pool, k, v, src_token_stride, slots, n_rows, stream);
  else if (pool.head_dim == 256)
    i8 ? launch_quantize_df<256, kInt8>(pool, k, v, src_token_stride, slots, n_rows, stream)
       : launch_quantize_df<256, kE4M3>(pool, k, v, src_token_stride, slots, n_rows, stream);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_reconstruct(const PoolView& pool, const int32_t* prefix_rows, int32_t n_prefix,
                              uint16_t* ws_k, uint16_t* ws_v, hipStream_t stream) {
  const int64_t n_rows = (int64_t)n_prefix * 2 * pool.n_kv_heads;
  if (n_rows == 0) return hipSuccess;
  if (pool.head_dim != kHeadDim) return hipErrorInvalidValue;
  const int64_t blocks = (n_rows + kRowsPerBlock - 1) / kRowsPerBlock;
  auto kernel = pool.format == kInt8 ? reconstruct_kernel<kInt8> : reconstruct_kernel<kE4M3>;
  hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(kBlock), 0, stream, pool.k_codes, pool.v_codes,
                     pool.k_scales, pool.v_scales, pool.code_row_stride, pool.scale_row_stride, prefix_rows, n_rows,
                     pool.n_kv_heads, (uint32_t)(pool.num_rows - 1), ws_k, ws_v);
  return hipGetLastError();
}

}  // namespace fp8kv
