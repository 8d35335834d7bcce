// decode.hip -- split-K GQA decode attention over the page-size-1 FP8 row pool.
//
// FreeToken PR #897 "perf(attention): add packed fp8 kv reads on gfx1201",
// description and "Fresh R9700 stage-1 A/B": a first stage computes one
// partial per (head group, split) over FP8 rows fetched through the row table
// (page size 1, randomized physical slots) and a merge kernel combines the
// partials.  FreeToken PR #853 "What changes": per-row FP32 scales.
//
// gfx950 design (not the pages' RDNA4 kernel):
//  * A workgroup (8 waves) covers one split of one (request, KV head); a wave
//    takes two 32-key steps at a time.  The request length is read with a
//    vector load next to the first (speculative, host-bounded) table read, so
//    it costs no extra round trip, and no code byte past the length's 64-key
//    group is fetched.
//  * Every lane loads exactly the code bytes its MFMA operands need, straight
//    into registers: for keys on the MFMA rows, 16-byte K chunks; for the P*V
//    contraction, 8 bytes of V per key, 16 lanes covering one whole 128-byte V
//    row.  All loads of both steps are in flight before the first wait; only
//    row indices and scales pass through LDS.
//  * QK^T runs on the bf16 MFMA 16x16x32 with E4M3 codes widened exactly to
//    bf16.  S^T = K * Q^T puts keys on the MFMA rows and the G query heads of
//    the group on the columns, so each lane holds 8 keys of one head: the
//    per-head maximum needs two cross-lane steps, and those 8 keys are exactly
//    the k-slots this lane feeds to the P*V MFMA, so P never moves between
//    lanes.  The per-row K scale and the softmax scale multiply the score tile
//    after the MFMA; the per-row V scale is folded into P.
//  * Online softmax in log2 units with a lazy maximum: the running maximum
//    moves (and O is rescaled) only when a step's maximum exceeds it by more
//    than 8, so p stays below 2^8 and most steps skip the rescale.
//  * Waves merge through LDS; one (o, log2-sum-exp) partial per split.

#include <math.h>

#include <type_traits>

#include "fp8kv_device.h"

namespace fp8kv {

namespace {

constexpr int kBlock = kDecodeWaves * kWave;
constexpr int kGroupKeys = kDecodeTilesPerWave * kDecodeTileKeys;  // keys a wave loads at once
// Row indices and scales are loaded one key per lane; a 32-key group leaves
// the upper half-wave reading duplicates into padding.
constexpr int kRowSlots = (kGroupKeys + kWave - 1) / kWave;
static_assert(kGroupKeys % kWave == 0 || kGroupKeys == kWave / 2, "a group covers whole or half waves of row indices");
static_assert(kDecodeTilesPerWave >= 1 && kDecodeTilesPerWave <= 4, "up to four steps in flight per wave");
constexpr float kLazyMaxSlack = 8.0f;  // log2 units: p <= 2^8 between rescales
constexpr float kLog2e = 1.4426950408889634f;

// Key order inside a 32-key step: k-group j of the P*V contraction holds keys
// 4j..4j+3 (first 16-key MFMA block) and 16+4j..16+4j+3 (second block).
__device__ __forceinline__ int step_key(int j, int r) { return (r < 4) ? 4 * j + r : 12 + 4 * j + r; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int G>
__global__ __launch_bounds__(kBlock) void decode_stage1_kernel(
    const uint8_t* __restrict__ k_codes, const uint8_t* __restrict__ v_codes,
    const float* __restrict__ k_scales, const float* __restrict__ v_scales, uint32_t code_row_stride,
    uint32_t scale_row_stride, const uint16_t* __restrict__ q, int32_t n_q_heads,
    const int32_t* __restrict__ table, int64_t table_stride, const int32_t* __restrict__ seq_lens,
    int32_t max_seq_len, int32_t n_split, int32_t chunk, int32_t split_stride, float qk_scale_log2,
    int32_t key_trim, uint32_t max_row, int32_t* __restrict__ header, float* __restrict__ part_o,
    float* __restrict__ part_lse) {
  static_assert(G >= 1 && G <= 16, "query heads per KV head must fit one 16-wide MFMA tile");
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int n = lane & 15;
  const int j = lane >> 4;
  const int split = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int key_begin = split * chunk;
  const int key_bound = min(key_begin + chunk, max_seq_len);  // host-side bound on this split's keys
  const int h0 = g * G;

  // The request length as a vector load, issued first: a scalar load would
  // share its wait with the kernel-argument loads and delay the table read.
  int b_lane = b;
  asm volatile("" : "+v"(b_lane));
  const int len_lane = seq_lens[b_lane];

  __shared__ __attribute__((aligned(16))) int32_t s_rows[kDecodeWaves][kRowSlots * kWave];
  __shared__ __attribute__((aligned(16))) float2 s_sc[kDecodeWaves][kRowSlots * kWave];
  __shared__ __attribute__((aligned(16))) float sm_o[kDecodeWaves][G][kHeadDim];
  __shared__ float sm_m[kDecodeWaves][16];
  __shared__ float sm_l[kDecodeWaves][16];

  const int32_t* trow = table + (int64_t)b * table_stride;
  // Row indices of the first group, read up to the host-side bound before the
  // length is known.  Every table entry below max_seq_len names a valid row
  // (padding included), so reading past the request's length is harmless.
  // They go to LDS before the length is used, which keeps the compiler from
  // sinking the read below the length's wait.
  int k0 = key_begin + wave * kGroupKeys;
  int rows_in[kRowSlots];
#pragma unroll
  for (int c = 0; c < kRowSlots; ++c) rows_in[c] = (int)min((uint32_t)trow[min(k0 + c * kWave + lane, key_bound - 1)], max_row);
#pragma unroll
  for (int c = 0; c < kRowSlots; ++c) s_rows[wave][c * kWave + lane] = rows_in[c];

  // Q^T operand: column n = query head h0 + n; for MFMA kk the lane's eight
  // k-slots are d = 64*(kk/2) + 16*j + 8*(kk%2) + [0, 8).
  // Columns n >= G repeat head G-1: MFMA outputs never mix columns, so they
  // only produce values that are never stored, and the loads need no branch
  // (which would make the waits on the loads issued before them inexact).
  bf16x8 qb[4];
  const uint16_t* qrow = q + ((int64_t)b * n_q_heads + h0 + min(n, G - 1)) * kHeadDim + 16 * j;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) qb[kk] = u4_as_bf16x8(*reinterpret_cast<const uint4*>(qrow + 64 * (kk >> 1) + 8 * (kk & 1)));

  const int L = __builtin_amdgcn_readfirstlane(len_lane) - key_trim;  // keys this stage covers
  const int key_end = min(key_begin + chunk, L);

  // Code addresses: row * stride (32 x 32 -> 64-bit) + the lane's bytes.  The
  // offsets stay on the global pointers so the loads are global, not flat.
  // K: key n of a 16-key block, 16-byte chunks j and 4+j.  V: 8 bytes at d = 8n.
  const uint8_t* kbase = k_codes + g * kHeadDim + 16 * j;
  const uint8_t* vbase = v_codes + g * kHeadDim + 8 * n;

  float m_run = -INFINITY;  // running (lazy) max, log2 units, of head n
  float l_part = 0.0f;      // sum of p for head n over this lane's keys
  f32x4 o[8];               // O[head 4j+i][d = 8n + nb]
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (bool first = true; k0 < key_end; k0 += kDecodeWaves * kGroupKeys, first = false) {
    // 1. Row indices of the group's keys through LDS (per-wave region).
    if (!first) {
#pragma unroll
      for (int c = 0; c < kRowSlots; ++c) {
        rows_in[c] = (int)min((uint32_t)trow[min(k0 + c * kWave + lane, key_bound - 1)], max_row);
        s_rows[wave][c * kWave + lane] = rows_in[c];
      }
    }
    __builtin_amdgcn_wave_barrier();

    // 2. Scale loads, issued before the code loads: loads complete in issue
    //    order, so writing the scales to LDS waits for them alone.
    float ksc[kRowSlots], vsc[kRowSlots];
#pragma unroll
    for (int c = 0; c < kRowSlots; ++c) {
      const uint32_t row = (uint32_t)rows_in[c];
      const uint64_t off = (uint64_t)row * scale_row_stride + g;
      ksc[c] = k_scales[off];
      vsc[c] = v_scales[off];
    }
    __builtin_amdgcn_sched_barrier(0);

    // 3. Every code load of the group, in step order.
    u32x4 kr[kDecodeTilesPerWave][4];
    uint2 vr[kDecodeTilesPerWave][8];
#pragma unroll
    for (int t = 0; t < kDecodeTilesPerWave; ++t) {
      const int32_t* rw = &s_rows[wave][t * kDecodeTileKeys];
      const uint64_t r0 = (uint64_t)(uint32_t)rw[n] * code_row_stride;
      const uint64_t r1 = (uint64_t)(uint32_t)rw[16 + n] * code_row_stride;
      kr[t][0] = *reinterpret_cast<const u32x4*>(kbase + r0);
      kr[t][1] = *reinterpret_cast<const u32x4*>(kbase + r0 + 64);
      kr[t][2] = *reinterpret_cast<const u32x4*>(kbase + r1);
      kr[t][3] = *reinterpret_cast<const u32x4*>(kbase + r1 + 64);
      const int4 va = *reinterpret_cast<const int4*>(rw + 4 * j);
      const int4 vb = *reinterpret_cast<const int4*>(rw + 16 + 4 * j);
      const int vrow[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
#pragma unroll
      for (int r = 0; r < 8; ++r)
        vr[t][r] = *reinterpret_cast<const uint2*>(vbase + (uint64_t)(uint32_t)vrow[r] * code_row_stride);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < kRowSlots; ++c) s_sc[wave][c * kWave + lane] = make_float2(ksc[c], vsc[c]);
    __builtin_amdgcn_wave_barrier();
    const bool tail = k0 + kGroupKeys > key_end;  // wave-uniform: only a request's last group

    // One 32-key step; t is a compile-time constant so kr/vr stay in registers.
    // Steps are not skipped (no branch the loads could sink into); keys at or
    // past the length are masked out of the softmax.
    auto step = [&](auto tc) {
      constexpr int t = decltype(tc)::value;
      const int t0 = k0 + t * kDecodeTileKeys;
      // S^T = K * Q^T: lane (n, j) holds chunks j and 4+j of keys n (block 0)
      // and 16+n (block 1).
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
      s0 = mfma16x16x32(fp8x8_to_bf16x8(kr[t][0].x, kr[t][0].y), qb[0], s0);
      s0 = mfma16x16x32(fp8x8_to_bf16x8(kr[t][0].z, kr[t][0].w), qb[1], s0);
      s0 = mfma16x16x32(fp8x8_to_bf16x8(kr[t][1].x, kr[t][1].y), qb[2], s0);
      s0 = mfma16x16x32(fp8x8_to_bf16x8(kr[t][1].z, kr[t][1].w), qb[3], s0);
      s1 = mfma16x16x32(fp8x8_to_bf16x8(kr[t][2].x, kr[t][2].y), qb[0], s1);
      s1 = mfma16x16x32(fp8x8_to_bf16x8(kr[t][2].z, kr[t][2].w), qb[1], s1);
      s1 = mfma16x16x32(fp8x8_to_bf16x8(kr[t][3].x, kr[t][3].y), qb[2], s1);
      s1 = mfma16x16x32(fp8x8_to_bf16x8(kr[t][3].z, kr[t][3].w), qb[3], s1);
      const float2* scp = &s_sc[wave][t * kDecodeTileKeys];
      const float4 c01 = *reinterpret_cast<const float4*>(&scp[4 * j]);
      const float4 c23 = *reinterpret_cast<const float4*>(&scp[4 * j + 2]);
      const float4 c45 = *reinterpret_cast<const float4*>(&scp[16 + 4 * j]);
      const float4 c67 = *reinterpret_cast<const float4*>(&scp[16 + 4 * j + 2]);

      // Scores in log2 units for head n, keys step_key(j, r).
      float sv[8] = {s0[0] * c01.x, s0[1] * c01.z, s0[2] * c23.x, s0[3] * c23.z,
                     s1[0] * c45.x, s1[1] * c45.z, s1[2] * c67.x, s1[3] * c67.z};
#pragma unroll
      for (int r = 0; r < 8; ++r) sv[r] *= qk_scale_log2;
      if (tail) {
#pragma unroll
        for (int r = 0; r < 8; ++r) sv[r] = (t0 + step_key(j, r) < key_end) ? sv[r] : -INFINITY;
      }
      float tmax = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])), fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
      tmax = max_over_row_groups(tmax);

      // Lazy maximum: move it (and rescale O and l) only when this step's
      // maximum exceeds it by more than the slack; otherwise p <= 2^slack.  A
      // fully masked step has tmax = -inf and leaves the state untouched; the
      // group's first step always holds key k0 < key_end, so m_run is finite
      // before any fully masked step.
      if (__any(tmax > m_run + kLazyMaxSlack)) {
        const float m_new = fmaxf(m_run, tmax);
        const float alpha = fast_exp2(m_run - m_new);
        m_run = m_new;
        l_part *= alpha;
        float ai[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ai[i] = __shfl(alpha, 4 * j + i);
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
#pragma unroll
          for (int i = 0; i < 4; ++i) o[nb][i] *= ai[i];
        }
      }

      float p[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) p[r] = fast_exp2(sv[r] - m_run);
      l_part += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      // P' = p * v_scale as the bf16 A operand (row = head n, k-slots = keys).
      const uint4 pu = make_uint4(f32x2_to_bf16x2(p[0] * c01.y, p[1] * c01.w), f32x2_to_bf16x2(p[2] * c23.y, p[3] * c23.w),
                                  f32x2_to_bf16x2(p[4] * c45.y, p[5] * c45.w), f32x2_to_bf16x2(p[6] * c67.y, p[7] * c67.w));
      const bf16x8 pa = u4_as_bf16x8(pu);

      // 4. V operand for N-block nb: byte nb of each key's 8 bytes, i.e.
      //    V[key][d = 8n + nb] for the lane's 8 keys (byte-transposed in registers).
      uint32_t lo[8], hi[8];
      transpose4x4_bytes(vr[t][0].x, vr[t][1].x, vr[t][2].x, vr[t][3].x, lo[0], lo[1], lo[2], lo[3]);
      transpose4x4_bytes(vr[t][4].x, vr[t][5].x, vr[t][6].x, vr[t][7].x, hi[0], hi[1], hi[2], hi[3]);
      transpose4x4_bytes(vr[t][0].y, vr[t][1].y, vr[t][2].y, vr[t][3].y, lo[4], lo[5], lo[6], lo[7]);
      transpose4x4_bytes(vr[t][4].y, vr[t][5].y, vr[t][6].y, vr[t][7].y, hi[4], hi[5], hi[6], hi[7]);
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) o[nb] = mfma16x16x32(pa, fp8x8_to_bf16x8(lo[nb], hi[nb]), o[nb]);
    };
    step(std::integral_constant<int, 0>{});
    if constexpr (kDecodeTilesPerWave > 1) step(std::integral_constant<int, 1>{});
    if constexpr (kDecodeTilesPerWave > 2) step(std::integral_constant<int, 2>{});
    if constexpr (kDecodeTilesPerWave > 3) step(std::integral_constant<int, 3>{});
    __builtin_amdgcn_wave_barrier();  // this group's LDS is consumed before the next overwrites it
  }

  // Per-head totals of this wave.
  const float l_tot = sum_over_row_groups(l_part);

  if (j == 0) {
    sm_m[wave][n] = m_run;
    sm_l[wave][n] = l_tot;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int head = 4 * j + i;
    if (head < G) {
      float* dst = &sm_o[wave][head][8 * n];
      *reinterpret_cast<float4*>(dst) = make_float4(o[0][i], o[1][i], o[2][i], o[3][i]);
      *reinterpret_cast<float4*>(dst + 4) = make_float4(o[4][i], o[5][i], o[6][i], o[7][i]);
    }
  }
  __syncthreads();

  // Merge the waves of this workgroup into one partial per query head; a
  // thread produces 4 consecutive d of one head.
  for (int idx = threadIdx.x; idx < G * (kHeadDim / 4); idx += kBlock) {
    const int h = idx / (kHeadDim / 4);
    const int d = 4 * (idx % (kHeadDim / 4));
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) M = fmaxf(M, sm_m[w][h]);
    float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
    float den = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kDecodeWaves; ++w) {
        const float wt = fast_exp2(sm_m[w][h] - M);
        const float4 v = *reinterpret_cast<const float4*>(&sm_o[w][h][d]);
        num.x += wt * v.x;
        num.y += wt * v.y;
        num.z += wt * v.z;
        num.w += wt * v.w;
        den += wt * sm_l[w][h];
      }
    }
    const float inv = (den > 0.f) ? 1.0f / den : 0.0f;
    const int64_t ph = ((int64_t)b * n_q_heads + h0 + h) * split_stride + split;
    *reinterpret_cast<float4*>(part_o + ph * kHeadDim + d) = make_float4(num.x * inv, num.y * inv, num.z * inv, num.w * inv);
    if (d == 0) part_lse[ph] = (den > 0.f) ? M + log2f(den) : -INFINITY;
  }
  // The split count for a merge launched without one.  Written last: a branch
  // at the top would split the entry block and serialize the argument loads
  // ahead of the first table read.
  if (split == 0 && g == 0 && b == 0 && threadIdx.x == 0) header[0] = n_split;
}

// Stage 2: out[b][h] = sum_s 2^(lse_s - M) o_s / sum_s 2^(lse_s - M) over the
// splits of (b, h).  One workgroup per (request, query head); wave w takes
// splits w, w+4, ...: it loads their lse and o vectors together (clamped
// indices, no branches), keeps its own maximum, and the four waves combine
// through LDS -- a single memory round trip.
//
// With APPEND, wave 0 also takes the request's new token (position
// seq_lens[b] - 1, left out of stage 1): it quantizes the bf16 K and V rows of
// the head group exactly as the quantize-on-write kernel does (same codec
// functions), scores q against the decoded codes, and folds the token in as a
// single-key partial (o = s_v * decode(v), lse = the score).  The workgroup of
// the group's first query head writes the codes and scales to the token's row
// new_slots[b]; every load of the kernel is independent (one round trip).
constexpr int kMergeBlock = 256;
constexpr int kMergeWaves = kMergeBlock / kWave;
constexpr int kMergeBatch = 16;  // splits per wave loaded at once
static_assert(FP8KV_MAX_SPLITS_INTERNAL <= kMergeWaves * kMergeBatch * 4, "merge passes stay few");

struct AppendKernelArgs {
  const uint16_t* q;
  const uint16_t* k_new;
  const uint16_t* v_new;
  int64_t new_token_stride;
  const int32_t* new_slots;
  uint8_t* k_codes;
  uint8_t* v_codes;
  float* k_scales;
  float* v_scales;
  int64_t code_row_stride;
  int64_t scale_row_stride;
  int32_t n_kv_heads;
  uint32_t max_row;
  float qk_scale_log2;
};

template <bool APPEND>
__global__ __launch_bounds__(kMergeBlock) void decode_merge_kernel(const int32_t* __restrict__ header,
                                                                  const float* __restrict__ part_o,
                                                                  const float* __restrict__ part_lse,
                                                                  int32_t split_stride, int32_t n_split_arg,
                                                                  int32_t n_q_heads, AppendKernelArgs app,
                                                                  uint16_t* __restrict__ out) {
  __shared__ float s_m[kMergeWaves];
  __shared__ float s_den[kMergeWaves];
  __shared__ float2 s_acc[kMergeWaves][kWave];
  const int64_t bh = blockIdx.x;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int n_split = n_split_arg >= 0 ? n_split_arg : header[0];
  const float* lse_p = part_lse + bh * split_stride;
  const float* po = part_o + bh * split_stride * kHeadDim + 2 * lane;

  // The new token's inputs: its bf16 K/V pair at d = 2*lane, 2*lane + 1, and q.
  uint32_t k2 = 0u, v2 = 0u, q2 = 0u;
  int64_t slot = 0;
  int64_t b = 0, g = 0;
  if constexpr (APPEND) {
    b = bh / n_q_heads;
    const int h = (int)(bh % n_q_heads);
    g = h / (n_q_heads / app.n_kv_heads);
    if (wave == 0) {
      slot = min((uint32_t)app.new_slots[b], app.max_row);  // out-of-range slots are clamped, never followed
      k2 = *reinterpret_cast<const uint32_t*>(app.k_new + b * app.new_token_stride + g * kHeadDim + 2 * lane);
      v2 = *reinterpret_cast<const uint32_t*>(app.v_new + b * app.new_token_stride + g * kHeadDim + 2 * lane);
      q2 = *reinterpret_cast<const uint32_t*>(app.q + bh * kHeadDim + 2 * lane);
    }
  }

  float m_w = -INFINITY, den = 0.f;
  float2 acc = make_float2(0.f, 0.f);
  // One batch of splits: wave w takes splits base + w + 4i, loaded together
  // (clamped indices, no branches) and folded into (m_w, den, acc).
  float lr[kMergeBatch];
  float2 v[kMergeBatch];
  auto load_batch = [&](int base) {
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      const int sidx = min(base + wave + kMergeWaves * i, n_split - 1);
      lr[i] = lse_p[sidx];
      v[i] = *reinterpret_cast<const float2*>(po + (int64_t)sidx * kHeadDim);
    }
  };
  auto fold_batch = [&](int base) {
    float mx = m_w;
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      lr[i] = (base + wave + kMergeWaves * i < n_split) ? lr[i] : -INFINITY;
      mx = fmaxf(mx, lr[i]);
    }
    if (mx != -INFINITY) {
      const float a = __builtin_amdgcn_exp2f(m_w - mx);  // 0 when m_w is -inf
      acc.x *= a;
      acc.y *= a;
      den *= a;
      m_w = mx;
#pragma unroll
      for (int i = 0; i < kMergeBatch; ++i) {
        const float w = __builtin_amdgcn_exp2f(lr[i] - m_w);
        acc.x += w * v[i].x;
        acc.y += w * v[i].y;
        den += w;
      }
    }
  };
  load_batch(0);  // in flight while wave 0 quantizes and scores the new token

  float lse_new = -INFINITY;
  float2 o_new = make_float2(0.f, 0.f);
  if constexpr (APPEND) {
    if (wave == 0) {
      // Quantize the K and V rows (128 values over the wave, two per lane).
      const float kx0 = bf16lo_to_f32(k2), kx1 = bf16hi_to_f32(k2);
      const float vx0 = bf16lo_to_f32(v2), vx1 = bf16hi_to_f32(v2);
      const float ka = wave_max(fmaxf(fabsf(kx0), fabsf(kx1)));
      const float va = wave_max(fmaxf(fabsf(vx0), fabsf(vx1)));
      const float sk = e4m3_row_scale(ka), sv = e4m3_row_scale(va);
      const uint32_t kc = f32x2_to_fp8x2<false>(e4m3_prescaled(kx0, ka, sk), e4m3_prescaled(kx1, ka, sk), 0u);
      const uint32_t vc = f32x2_to_fp8x2<false>(e4m3_prescaled(vx0, va, sv), e4m3_prescaled(vx1, va, sv), 0u);
      // Score and value from the decoded codes, as stage 1 sees every other row.
      float kd[4], vd[4];
      fp8x4_to_f32x4(kc, kd);
      fp8x4_to_f32x4(vc, vd);
      const float dot = wave_sum(bf16lo_to_f32(q2) * kd[0] + bf16hi_to_f32(q2) * kd[1]);
      lse_new = dot * sk * app.qk_scale_log2;
      o_new = make_float2(vd[0] * sv, vd[1] * sv);
      // One workgroup per (request, KV head) stores the row.
      if ((bh % n_q_heads) % (n_q_heads / app.n_kv_heads) == 0) {
        *reinterpret_cast<uint16_t*>(app.k_codes + slot * app.code_row_stride + g * kHeadDim + 2 * lane) = (uint16_t)kc;
        *reinterpret_cast<uint16_t*>(app.v_codes + slot * app.code_row_stride + g * kHeadDim + 2 * lane) = (uint16_t)vc;
        if (lane == 0) {
          app.k_scales[slot * app.scale_row_stride + g] = sk;
          app.v_scales[slot * app.scale_row_stride + g] = sv;
        }
      }
    }
  }

  fold_batch(0);
  for (int base = kMergeWaves * kMergeBatch; base < n_split; base += kMergeWaves * kMergeBatch) {
    load_batch(base);
    fold_batch(base);
  }

  if constexpr (APPEND) {
    if (wave == 0) {  // the new token as one more single-key partial
      const float mx = fmaxf(m_w, lse_new);
      const float a = __builtin_amdgcn_exp2f(m_w - mx);
      const float w = __builtin_amdgcn_exp2f(lse_new - mx);
      acc.x = acc.x * a + w * o_new.x;
      acc.y = acc.y * a + w * o_new.y;
      den = den * a + w;
      m_w = mx;
    }
  }

  if (lane == 0) {
    s_m[wave] = m_w;
    s_den[wave] = den;
  }
  s_acc[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    float M = s_m[0];
#pragma unroll
    for (int w = 1; w < kMergeWaves; ++w) M = fmaxf(M, s_m[w]);
    float2 t = make_float2(0.f, 0.f);
    float d = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kMergeWaves; ++w) {
        const float a = __builtin_amdgcn_exp2f(s_m[w] - M);
        t.x += a * s_acc[w][lane].x;
        t.y += a * s_acc[w][lane].y;
        d += a * s_den[w];
      }
    }
    const float inv = (d > 0.f) ? 1.0f / d : 0.0f;
    *reinterpret_cast<uint32_t*>(out + bh * kHeadDim + 2 * lane) = f32x2_to_bf16x2(t.x * inv, t.y * inv);
  }
}

template <int G>
hipError_t launch_stage1_g(const PoolView& pool, const uint16_t* q, int32_t batch, int32_t n_q_heads,
                           const int32_t* row_table, int64_t table_stride, const int32_t* seq_lens,
                           int32_t max_seq_len, float qk_scale_log2, const DecodeGeometry& geo, const DecodeWorkspace& ws,
                           int32_t key_trim, hipStream_t stream) {
  dim3 grid((unsigned)geo.n_split, (unsigned)pool.n_kv_heads, (unsigned)batch);
  hipLaunchKernelGGL(decode_stage1_kernel<G>, grid, dim3(kBlock), 0, stream, pool.k_codes, pool.v_codes,
                     pool.k_scales, pool.v_scales, (uint32_t)pool.code_row_stride, (uint32_t)pool.scale_row_stride,
                     q, n_q_heads,
                     row_table, table_stride, seq_lens, max_seq_len, geo.n_split, geo.chunk, ws.split_stride,
                     qk_scale_log2, key_trim, (uint32_t)(pool.num_rows - 1), ws.header, ws.part_o, ws.part_lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_stage1(const PoolView& pool, const uint16_t* q, int32_t batch, int32_t n_q_heads,
                                const int32_t* row_table, int64_t table_stride, const int32_t* seq_lens,
                                int32_t max_seq_len, float sm_scale, const DecodeGeometry& geo, const DecodeWorkspace& ws,
                                int32_t key_trim, hipStream_t stream) {
  const float qk_scale_log2 = sm_scale * kLog2e;
  switch (n_q_heads / pool.n_kv_heads) {
    case 1: return launch_stage1_g<1>(pool, q, batch, n_q_heads, row_table, table_stride, seq_lens, max_seq_len, qk_scale_log2, geo, ws, key_trim, stream);
    case 2: return launch_stage1_g<2>(pool, q, batch, n_q_heads, row_table, table_stride, seq_lens, max_seq_len, qk_scale_log2, geo, ws, key_trim, stream);
    case 4: return launch_stage1_g<4>(pool, q, batch, n_q_heads, row_table, table_stride, seq_lens, max_seq_len, qk_scale_log2, geo, ws, key_trim, stream);
    case 8: return launch_stage1_g<8>(pool, q, batch, n_q_heads, row_table, table_stride, seq_lens, max_seq_len, qk_scale_log2, geo, ws, key_trim, stream);
    case 16: return launch_stage1_g<16>(pool, q, batch, n_q_heads, row_table, table_stride, seq_lens, max_seq_len, qk_scale_log2, geo, ws, key_trim, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_merge(int32_t batch, int32_t n_q_heads, const DecodeWorkspace& ws, int32_t n_split,
                               uint16_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(decode_merge_kernel<false>, dim3((unsigned)((int64_t)batch * n_q_heads)), dim3(kMergeBlock), 0,
                     stream, ws.header, ws.part_o, ws.part_lse, ws.split_stride, n_split, n_q_heads, AppendKernelArgs{},
                     out);
  return hipGetLastError();
}

hipError_t launch_decode_merge_append(const PoolView& pool, int32_t batch, int32_t n_q_heads, const DecodeWorkspace& ws,
                                      int32_t n_split, const AppendArgs& app, uint16_t* out, hipStream_t stream) {
  const AppendKernelArgs a{app.q, app.k_new, app.v_new, app.new_token_stride, app.new_slots,
                           pool.k_codes, pool.v_codes, pool.k_scales, pool.v_scales,
                           pool.code_row_stride, pool.scale_row_stride, pool.n_kv_heads,
                           (uint32_t)(pool.num_rows - 1), app.sm_scale * kLog2e};
  hipLaunchKernelGGL(decode_merge_kernel<true>, dim3((unsigned)((int64_t)batch * n_q_heads)), dim3(kMergeBlock), 0,
                     stream, ws.header, ws.part_o, ws.part_lse, ws.split_stride, n_split, n_q_heads, a, out);
  return hipGetLastError();
}

}  // namespace fp8kv
