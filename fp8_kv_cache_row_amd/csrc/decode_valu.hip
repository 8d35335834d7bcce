// decode_valu.hip -- a decode stage 1 that uses no matrix instructions: the
// plain-VALU counterpart of decode_stage1_kernel, kept so the choice of MFMA
// for the decode contraction can be measured on this hardware rather than
// asserted.
//
// FreeToken PR #897 "perf(attention): add packed fp8 kv reads on gfx1201",
// description and "Fresh R9700 stage-1 A/B": split-K stage 1 over FP8 rows
// fetched through a page-size-1 row table, one partial per (head group,
// split), combined by a merge kernel.  FreeToken PR #853 "What changes":
// per-row FP32 scales.
//
// Same grid, split choice and partial format as the MFMA stage 1 (so the
// same merge kernel combines it): a workgroup of 8 waves covers one split of
// one (request, KV head); a wave takes 64 keys at a time, one key per lane.
//  * QK^T: lane k loads its key's 128 E4M3 codes (eight 16-byte loads),
//    widens them to fp32 four at a time and accumulates the G dot products
//    against the group's query vectors, which sit in LDS as fp32 (every lane
//    reads the same address: broadcast).
//  * Online softmax per query head over the wave's 64 keys (DPP reductions).
//  * P*V: the wave stages its 64 V rows in LDS (8 KB) and the probabilities
//    (times the V row scale) beside them; lane l then owns d = 2l, 2l+1 and
//    accumulates the G output vectors over the 64 keys.
//  * The 8 waves merge through LDS into one (o, log2-sum-exp) partial per
//    (request, query head, split).
#include <math.h>

#include "fp8kv_device.h"

namespace fp8kv {

namespace {

constexpr int kVWaves = 8;
constexpr int kVBlock = kVWaves * kWave;
constexpr int kVKeys = kWave;  // keys per wave and pass: one per lane
constexpr float kVNoMax = -1.0e30f;

template <int G>
struct ValuLds {
  float q[G][kHeadDim];                          // query vectors of the group, fp32
  float p[kVWaves][kVKeys][G];                   // p * v_scale per (key, head)
  union {
    uint8_t v[kVWaves][kVKeys][kHeadDim];        // staged V codes of each wave's keys
    float o[kVWaves][G][kHeadDim];               // per-wave outputs for the workgroup merge
  } u;
  float m[kVWaves][G];
  float l[kVWaves][G];
};

template <int G>
__global__ __launch_bounds__(kVBlock) void decode_stage1_valu_kernel(
    const uint8_t* __restrict__ k_codes, const uint8_t* __restrict__ v_codes, const float* __restrict__ k_scales,
    const float* __restrict__ v_scales, uint32_t code_row_stride, uint32_t scale_row_stride,
    const uint16_t* __restrict__ q, int32_t n_q_heads, const int32_t* __restrict__ table, int64_t table_stride,
    const int32_t* __restrict__ seq_lens, int32_t max_seq_len, int32_t n_split, int32_t chunk, int32_t split_stride,
    float qk_scale_log2, uint32_t max_row, int32_t* __restrict__ header, float* __restrict__ part_o,
    float* __restrict__ part_lse) {
  static_assert(sizeof(ValuLds<G>) <= 160 * 1024, "LDS");
  __shared__ ValuLds<G> s;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  // Grid (8 * Hkv, ceil(n_split / 8), batch), as the MFMA stage 1: workgroup
  // x + 8 Hkv (y + Y z) runs split 8y + (x & 7) of KV head x >> 3.
  const int split_raw = 8 * (int)blockIdx.y + (int)(blockIdx.x & 7u);
  const bool owner = split_raw < n_split;
  const int split = min(split_raw, n_split - 1);
  const int g = (int)(blockIdx.x >> 3);
  const int b = (int)blockIdx.z;
  const int h0 = g * G;

  for (int idx = threadIdx.x; idx < G * kHeadDim; idx += kVBlock) {
    const int hh = idx / kHeadDim, d = idx - hh * kHeadDim;
    const uint16_t bits = q[((int64_t)b * n_q_heads + h0 + hh) * kHeadDim + d];
    s.q[hh][d] = __uint_as_float((uint32_t)bits << 16);
  }
  __syncthreads();

  const int len = min(seq_lens[b], max_seq_len);
  const int key_begin = split * chunk;
  const int key_end = min(key_begin + chunk, len);
  const int32_t* trow = table + (int64_t)b * table_stride;

  float m_run[G], l_run[G], o[G][2];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    m_run[hh] = kVNoMax;
    l_run[hh] = 0.f;
    o[hh][0] = o[hh][1] = 0.f;
  }

  for (int k0 = key_begin + wave * kVKeys; k0 < key_end; k0 += kVWaves * kVKeys) {
    const int key = k0 + lane;
    const bool live = key < key_end;
    const uint32_t row = min((uint32_t)trow[min(key, key_end - 1)], max_row);
    const uint64_t soff = (uint64_t)row * scale_row_stride + g;
    const float ks = k_scales[soff];
    const float vs = v_scales[soff];
    const uint8_t* krow = k_codes + (uint64_t)row * code_row_stride + g * kHeadDim;
    const uint8_t* vrow = v_codes + (uint64_t)row * code_row_stride + g * kHeadDim;
    // stage this key's V row for the P*V pass
    uint4 vv[kHeadDim / 16];
#pragma unroll
    for (int c = 0; c < kHeadDim / 16; ++c) vv[c] = *reinterpret_cast<const uint4*>(vrow + 16 * c);
    // scores: G dot products of the key's codes with the query vectors
    float acc[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) acc[hh] = 0.f;
#pragma unroll
    for (int c = 0; c < kHeadDim / 16; ++c) {
      const uint4 w = *reinterpret_cast<const uint4*>(krow + 16 * c);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float kf[4];
        fp8x4_to_f32x4(ww[e], kf);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int d = 16 * c + 4 * e + t;
#pragma unroll
          for (int hh = 0; hh < G; ++hh) acc[hh] = fmaf(kf[t], s.q[hh][d], acc[hh]);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < kHeadDim / 16; ++c) *reinterpret_cast<uint4*>(&s.u.v[wave][lane][16 * c]) = vv[c];

    // online softmax per head over the wave's 64 keys (log2 units)
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float sc = live ? acc[hh] * ks * qk_scale_log2 : -INFINITY;
      const float m_new = fmaxf(m_run[hh], wave_max(sc));
      const float alpha = __builtin_amdgcn_exp2f(m_run[hh] - m_new);
      const float p = __builtin_amdgcn_exp2f(sc - m_new);
      m_run[hh] = m_new;
      l_run[hh] = l_run[hh] * alpha + wave_sum(p);
      o[hh][0] *= alpha;
      o[hh][1] *= alpha;
      s.p[wave][lane][hh] = p * vs;
    }
    __builtin_amdgcn_wave_barrier();
    // P*V: lane owns d = 2 lane, 2 lane + 1
    for (int kk = 0; kk < kVKeys; ++kk) {
      const uint32_t pair = *reinterpret_cast<const uint16_t*>(&s.u.v[wave][kk][2 * lane]);
      const f32x2 vf = __builtin_amdgcn_cvt_pk_f32_fp8(pair, false);
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float pk = s.p[wave][kk][hh];
        o[hh][0] = fmaf(pk, vf.x, o[hh][0]);
        o[hh][1] = fmaf(pk, vf.y, o[hh][1]);
      }
    }
    __builtin_amdgcn_wave_barrier();  // the wave's staging area is read before the next pass overwrites it
  }

  // merge the 8 waves into one partial per head
  __syncthreads();  // every wave is done with its V staging (shared with the merge area)
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    if (lane == 0) {
      s.m[wave][hh] = m_run[hh];
      s.l[wave][hh] = l_run[hh];
    }
    s.u.o[wave][hh][2 * lane] = o[hh][0];
    s.u.o[wave][hh][2 * lane + 1] = o[hh][1];
  }
  __syncthreads();
  if (owner) {
    for (int idx = threadIdx.x; idx < G * kHeadDim; idx += kVBlock) {
      const int hh = idx / kHeadDim, d = idx - hh * kHeadDim;
      float M = s.m[0][hh];
#pragma unroll
      for (int w = 1; w < kVWaves; ++w) M = fmaxf(M, s.m[w][hh]);
      float num = 0.f, den = 0.f;
#pragma unroll
      for (int w = 0; w < kVWaves; ++w) {
        const float wt = __builtin_amdgcn_exp2f(s.m[w][hh] - M);
        num = fmaf(wt, s.u.o[w][hh][d], num);
        den = fmaf(wt, s.l[w][hh], den);
      }
      const int64_t ph = ((int64_t)b * n_q_heads + h0 + hh) * split_stride + split;
      part_o[ph * kHeadDim + d] = den > 0.f ? num / den : 0.f;
      if (d == 0) part_lse[ph] = den > 0.f ? M + log2f(den) : -INFINITY;
    }
  }
  if (split == 0 && g == 0 && b == 0 && threadIdx.x == 0) header[0] = n_split;
}

template <int G>
hipError_t launch_valu_g(const PoolView& pool, const uint16_t* q, const DecodeShape& sh, float qk,
                         const DecodeGeometry& geo, const DecodeWorkspace& ws, hipStream_t stream) {
  const dim3 grid((unsigned)(8 * pool.n_kv_heads), (unsigned)((geo.n_split + 7) / 8), (unsigned)sh.batch);
  hipLaunchKernelGGL(decode_stage1_valu_kernel<G>, grid, dim3(kVBlock), 0, stream, pool.k_codes, pool.v_codes,
                     pool.k_scales, pool.v_scales, (uint32_t)pool.code_row_stride, (uint32_t)pool.scale_row_stride, q,
                     sh.n_q_heads, sh.row_table, sh.table_stride, sh.seq_lens, sh.max_seq_len, geo.n_split, geo.chunk,
                     ws.split_stride, qk, (uint32_t)(pool.num_rows - 1), ws.header, ws.part_o, ws.part_lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_stage1_valu(const PoolView& pool, const uint16_t* q, const DecodeShape& sh, float sm_scale,
                                     const DecodeGeometry& geo, const DecodeWorkspace& ws, hipStream_t stream) {
  if (pool.head_dim != kHeadDim || pool.format != kE4M3 || sh.n_qrows != 1 || sh.window != 0)
    return hipErrorInvalidValue;
  if (sh.batch > FP8KV_MAX_DECODE_GROUPS_INTERNAL) return hipErrorInvalidValue;
  const float qk = sm_scale * 1.4426950408889634f;
  switch (sh.n_q_heads / pool.n_kv_heads) {
    case 1: return launch_valu_g<1>(pool, q, sh, qk, geo, ws, stream);
    case 2: return launch_valu_g<2>(pool, q, sh, qk, geo, ws, stream);
    case 4: return launch_valu_g<4>(pool, q, sh, qk, geo, ws, stream);
    case 8: return launch_valu_g<8>(pool, q, sh, qk, geo, ws, stream);
    case 16: return launch_valu_g<16>(pool, q, sh, qk, geo, ws, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fp8kv
