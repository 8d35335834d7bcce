// read_floor.hip -- measurement kernels for the benchmark, not part of the
// FP8 KV path: what one launch can read from HBM on this machine, so the
// decode kernels' bandwidth can be set against a floor measured the same way
// (cold buffers rotated, HIP graph replay) rather than only the published peak.
//
//  * fp8kv_floor_read: a contiguous read of `bytes` bytes, 16 bytes per lane
//    and eight loads in flight per lane, every loaded word folded into a
//    checksum (stored only if it equals an unlikely value, so the loads stay).
//  * Both use non-temporal loads (the lines are not kept for reuse), which
//    read a cold buffer from HBM ~10 % faster than plain loads here.
//  * fp8kv_floor_gather: whole row records of `record_bytes` bytes (at most
//    2 KB) read through a row table -- every byte a page-size-1 reader of
//    those rows must fetch, in table order, each record by consecutive lanes,
//    16 records in flight per wave.
//
// Plain C ABI (device pointers, sizes, a hipStream_t as void*); 0 on success,
// 1 for invalid sizes or pointers, 2 when the launch fails.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kBlock = 512;
constexpr int kUnroll = 8;
constexpr uint32_t kNever = 0x9E3779B9u;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__global__ __launch_bounds__(kBlock) void read_contiguous(const uint4* __restrict__ p, int64_t n_vec,
                                                          uint32_t* __restrict__ sink) {
  int64_t i = (int64_t)blockIdx.x * kBlock * kUnroll + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * kBlock * kUnroll;
  uint32_t acc = 0;
  for (; i < n_vec; i += stride) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t k = i + (int64_t)u * kBlock;
      v[u] = k < n_vec ? load_nt(p + k) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == kNever) sink[0] = acc;
}

// A wave takes kGatherKeys consecutive table entries and reads their whole
// records: lane l loads 16-byte chunks l, l + 64, ... of each record, so every
// load instruction reads up to 1 KB of one record contiguously, and all of the
// wave's loads are issued before the first is used.
constexpr int kGatherKeys = 16;
constexpr int kMaxChunks = 2;  // records of up to 2 x 64 x 16 = 2 KB

__global__ __launch_bounds__(kBlock) void read_records(const uint8_t* __restrict__ pool, int64_t num_records,
                                                       int32_t rec_vec, const int32_t* __restrict__ table,
                                                       int32_t n_keys, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int waves_total = gridDim.x * (kBlock / 64);
  uint32_t acc = 0;
  for (int k0 = ((int)blockIdx.x * (kBlock / 64) + wave) * kGatherKeys; k0 < n_keys;
       k0 += waves_total * kGatherKeys) {
    const int my = min(k0 + (lane & (kGatherKeys - 1)), n_keys - 1);
    const int row_lane = (int)min((int64_t)(uint32_t)table[my], num_records - 1);
    uint4 v[kGatherKeys][kMaxChunks];
#pragma unroll
    for (int u = 0; u < kGatherKeys; ++u) {
      const int row = __builtin_amdgcn_readlane(row_lane, u);
      const uint4* rec = reinterpret_cast<const uint4*>(pool + (int64_t)row * rec_vec * 16);
      const bool key_ok = k0 + u < n_keys;
#pragma unroll
      for (int c = 0; c < kMaxChunks; ++c) {
        const int chunk = lane + 64 * c;
        v[u][c] = (key_ok && chunk < rec_vec) ? load_nt(rec + chunk) : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < kGatherKeys; ++u)
#pragma unroll
      for (int c = 0; c < kMaxChunks; ++c) acc ^= v[u][c].x ^ v[u][c].y ^ v[u][c].z ^ v[u][c].w;
  }
  if (acc == kNever) sink[0] = acc;
}

}  // namespace

extern "C" {

int fp8kv_floor_read(const void* buf, int64_t bytes, int32_t grid, uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes <= 0 || bytes % 16 != 0 || grid <= 0) return 1;
  hipLaunchKernelGGL(read_contiguous, dim3((unsigned)grid), dim3(kBlock), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(buf), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

int fp8kv_floor_gather(const void* pool, int64_t num_records, int64_t record_bytes, const int32_t* table,
                       int32_t n_keys, int32_t grid, uint32_t* sink, void* stream) {
  if (!pool || !table || !sink || num_records <= 0 || record_bytes <= 0 || record_bytes % 16 != 0 || n_keys <= 0 ||
      grid <= 0 || record_bytes > 16 * 64 * kMaxChunks)
    return 1;
  hipLaunchKernelGGL(read_records, dim3((unsigned)grid), dim3(kBlock), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint8_t*>(pool), num_records, (int32_t)(record_bytes / 16), table, n_keys,
                     sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
