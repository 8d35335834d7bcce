// prefill.hip -- causal chunked-prefill attention over [bf16 workspace prefix ;
// bf16 current chunk] on the gfx950 bf16 MFMA.
//
// FreeToken PR #853 "opt-in FP8 KV cache", "What changes": historical FP8 rows
// are reconstructed once per layer into one shared BF16 workspace and the
// current chunk's K/V stay BF16; "Paired end-to-end A/B": the 8K
// historical-prefix + 8K new-token operator.
//
// Work decomposition: a workgroup owns 256 "query rows", each one
// (query token, query head) pair of a single KV head's group (256/G tokens x
// G heads), so one K/V tile staged in LDS feeds every query head of the
// group.  Eight waves take 32 rows each as two 16-row blocks, which share
// every K and V operand read from LDS.  Per 32-key sub-step a wave computes
// S^T = K * Q^T (keys on MFMA rows, query rows on columns) so that a lane holds
// 8 keys of one query row: the row max needs two cross-lane steps (gfx950 row
// swaps), and the same registers are the k-slots of the P*V MFMA.
//
// K and V tiles (64 keys) are both stored row-major, [key][16 chunks of
// 16 B], chunk c of key m at position c ^ (m & 15) for K and c ^ (2m & 15)
// for V (each conflict-free for the reads it serves).  They are fetched by
// global-to-LDS loads, which write lane l's 16 bytes at LDS offset 16 l of the
// instruction's 1 KB (4 key rows): lane l fetches chunk (l & 15) ^ (key & 15)
// of its key, so the swizzle comes from the gather and no data passes through
// registers.  The P*V operand (V[key][d] for 4 consecutive keys at one d) is
// read with the gfx950 transposing LDS read: within a 16-lane group, source
// lane s names row s/4, columns 4(s%4)..+3 of a 4x16 block, and lane i
// receives column i of its 4 rows.
//
// Pipelining: the tiles are double-buffered, each buffer its own LDS object;
// the loads of tile t+1 are issued right after the barrier that opens tile t,
// so one barrier per tile suffices and the load latency hides behind the MFMA
// work.
//
// Softmax in log2 units against a fixed reference per query row: the maximum
// of the row's first 32 keys (key 0 is among them and every row sees it).
// p = 2^(s - ref) is never rescaled, so between the first sub-step and the
// end the accumulators are touched by the MFMAs alone -- no rescale branch,
// and none of the register copies the compiler places at such a branch's
// join (measured: 1.46 against 1.70 ms for the 8K + 8K operator).  Any key
// far enough above the reference to overflow p, the row sum or O leaves a
// non-finite value behind (inf and NaN absorb), so a workgroup whose l and O
// are finite got the result a running maximum gives, up to rounding; one that
// is not runs its tiles again with a lazy running maximum (O and l rescaled
// when a sub-step's maximum passes the running one by more than 8).  The row
// sums are an MFMA of P against a block of ones, which also normalizes by
// exactly the bf16 p that P*V uses.  Workgroups with the most keys (the last
// query tokens) are launched first.
#include <math.h>

#include <type_traits>

#include "fp8kv_device.h"

namespace fp8kv {

namespace {

// 32 query rows per wave (two 16-row blocks share every K/V operand read),
// 256 rows per workgroup, two waves per SIMD (under 256 registers, no spills).
// Measured on the 8K + 8K operator against 16 rows per wave at four waves
// per SIMD: 2.06 vs 2.13-2.20 ms.
#ifndef FP8KV_PREFILL_ROW_BLOCKS
#define FP8KV_PREFILL_ROW_BLOCKS 2
#endif
#ifndef FP8KV_PREFILL_ROWS
#define FP8KV_PREFILL_ROWS 256
#endif
#ifndef FP8KV_PREFILL_WAVES_PER_EU
#define FP8KV_PREFILL_WAVES_PER_EU 2
#endif
constexpr int kRowBlocks = FP8KV_PREFILL_ROW_BLOCKS;    // 16-row query blocks per wave
constexpr int kRowsPerWg = FP8KV_PREFILL_ROWS;
constexpr int kWaves = kRowsPerWg / (16 * kRowBlocks);
constexpr int kBlock = kWaves * kWave;
constexpr int kTileKeys = 64;
constexpr int kRowBytes = kHeadDim * 2;                 // one bf16 key row
constexpr int kTileBytes = kTileKeys * kRowBytes;       // 16 KB per tile
constexpr int kLoadsPerWave = kTileKeys / 4 / kWaves;   // 1 KB (4 rows) per load
constexpr float kLazyMaxSlack = 8.0f;
static_assert(kLoadsPerWave >= 1 && kLoadsPerWave * 4 * kWaves == kTileKeys, "a tile is whole 4-row loads");

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Byte offset of 16-byte chunk c of key m (tile-local) in a K tile: position
// c ^ (m & 15), so the 16 keys of one QK^T operand read (same chunk) hit 16
// different positions.
__device__ __forceinline__ int chunk_at(int m, int c) { return m * kRowBytes + ((c ^ (m & 15)) << 4); }
// The same for a V tile, position c ^ (2m & 15): one transposing read takes
// chunks 2nb and 2nb+1 of 8 consecutive keys, and doubling the key keeps the
// 8 position pairs {x, x ^ 1} apart.
__device__ __forceinline__ int vswz(int m) { return (2 * m) & 15; }
__device__ __forceinline__ int vchunk_at(int m, int c) { return m * kRowBytes + ((c ^ vswz(m)) << 4); }

__device__ __forceinline__ void g2lds16(const uint16_t* g, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

__device__ __forceinline__ uint2 ds_read_tr16(const uint8_t* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
  return __builtin_bit_cast(uint2, v);
}

template <int G>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(FP8KV_PREFILL_WAVES_PER_EU))) void prefill_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ ws_k, const uint16_t* __restrict__ ws_v,
    const uint16_t* __restrict__ k_cur, const uint16_t* __restrict__ v_cur, int32_t n_prefix, int32_t n_tokens,
    int32_t n_q_heads, int32_t n_kv_heads, float qk_scale_log2, uint16_t* __restrict__ out) {
  constexpr int BQ = kRowsPerWg / G;  // query tokens per workgroup
  // One LDS object per buffer: the compiler then knows that the loads filling
  // one buffer never write what the reads of the other see, and keeps the
  // next tile's loads in flight while this tile is computed (with a single
  // two-buffer array it waited for them before this tile's first LDS read).
  __shared__ __attribute__((aligned(16))) uint8_t k_lds0[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t k_lds1[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t v_lds0[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t v_lds1[kTileBytes];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int n = lane & 15;
  const int j = lane >> 4;
  const int g = blockIdx.y;
  const int h0 = g * G;
  const int i0 = (gridDim.x - 1 - blockIdx.x) * BQ;  // most keys first
  const int i_last = min(i0 + BQ, n_tokens) - 1;
  const int n_keys = n_prefix + i_last + 1;  // keys any row of this workgroup may see

  // Q^T operand for the wave's 16-row column blocks; rows past the chunk
  // reuse the last token (never stored).
  bf16x8 qb[kRowBlocks][4];
  int row_tok[kRowBlocks];
#pragma unroll
  for (int cb = 0; cb < kRowBlocks; ++cb) {
    const int rho = (wave * kRowBlocks + cb) * 16 + n;
    const int tok = min(i0 + rho / G, n_tokens - 1);
    const int head = h0 + rho % G;
    row_tok[cb] = tok;
    const uint16_t* qp = q + ((int64_t)tok * n_q_heads + head) * kHeadDim + 8 * j;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qb[cb][kk] = u4_as_bf16x8(*reinterpret_cast<const uint4*>(qp + 32 * kk));
  }

  float m_run[kRowBlocks];  // softmax reference of row n (log2 units)
  f32x4 o[kRowBlocks][8];   // O[row 4j+i][d = 16nb + n]
  f32x4 lsum[kRowBlocks];   // row sums of bf16(p) (an MFMA against ones): row 4j+i in slot i
#pragma unroll
  for (int mb = 0; mb < kRowBlocks; ++mb) {
    m_run[mb] = -INFINITY;
    lsum[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) o[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // Four registers of bf16 ones for the row-sum MFMA.  The empty asm hides
  // that the four are equal; otherwise the compiler keeps one and rebuilds the
  // other three with a move each before every row-sum MFMA.
  uint4 ones_u = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);
  asm volatile("" : "+v"(ones_u.x), "+v"(ones_u.y), "+v"(ones_u.z), "+v"(ones_u.w));
  const bf16x8 ones = u4_as_bf16x8(ones_u);

  const int64_t kv_row = (int64_t)n_kv_heads * kHeadDim;  // elements between tokens
  const int n_tiles = (n_keys + kTileKeys - 1) / kTileKeys;
  // first key index at which any row of this workgroup needs the causal mask
  const int diag = n_prefix + i0;

  // This lane's share of a tile fetch: load i covers tile-local keys
  // 4(kLoadsPerWave * wave + i) + [0, 4); the lane takes key +(lane >> 4) and
  // the chunk that lands at position (lane & 15) of that key's row.
  // Offsets are unsigned 32-bit bytes from a wave-uniform tile base, so each
  // load is a scalar base plus one 32-bit lane offset.
  int fkey[kLoadsPerWave];
  uint32_t fofs[kLoadsPerWave], vfofs[kLoadsPerWave];
#pragma unroll
  for (int i = 0; i < kLoadsPerWave; ++i) {
    fkey[i] = 4 * (kLoadsPerWave * wave + i) + (lane >> 4);
    fofs[i] = (uint32_t)(fkey[i] * (int)kv_row + g * kHeadDim + (((lane & 15) ^ (fkey[i] & 15)) << 3)) * 2u;
    vfofs[i] = (uint32_t)(fkey[i] * (int)kv_row + g * kHeadDim + (((lane & 15) ^ vswz(fkey[i])) << 3)) * 2u;
  }
  auto fetch = [&](auto bufc, int u0) {
    constexpr int buf = decltype(bufc)::value;
    uint8_t* kd = (buf == 0 ? k_lds0 : k_lds1) + kLoadsPerWave * wave * 1024;
    uint8_t* vd = (buf == 0 ? v_lds0 : v_lds1) + kLoadsPerWave * wave * 1024;
    if (u0 + kTileKeys <= n_prefix || (u0 >= n_prefix && u0 + kTileKeys <= n_keys)) {
      // the whole tile comes from one source: one base plus fixed offsets
      const int64_t base = (u0 < n_prefix) ? (int64_t)u0 * kv_row : (int64_t)(u0 - n_prefix) * kv_row;
      const uint16_t* kb = ((u0 < n_prefix) ? ws_k : k_cur) + base;
      const uint16_t* vb = ((u0 < n_prefix) ? ws_v : v_cur) + base;
#pragma unroll
      for (int i = 0; i < kLoadsPerWave; ++i) {
        g2lds16(reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(kb) + fofs[i]), kd + i * 1024);
        g2lds16(reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(vb) + vfofs[i]), vd + i * 1024);
      }
    } else {
      // straddles the workspace/chunk boundary or the last visible key; keys
      // past n_keys re-read the last one (masked, never weighted)
#pragma unroll
      for (int i = 0; i < kLoadsPerWave; ++i) {
        const int u = min(u0 + fkey[i], n_keys - 1);
        const int64_t off = (u < n_prefix) ? (int64_t)u * kv_row : (int64_t)(u - n_prefix) * kv_row;
        const int64_t klo = (int64_t)(fofs[i] / 2u) - fkey[i] * kv_row;  // head + chunk part (elements)
        const int64_t vlo = (int64_t)(vfofs[i] / 2u) - fkey[i] * kv_row;
        g2lds16(((u < n_prefix) ? ws_k : k_cur) + off + klo, kd + i * 1024);
        g2lds16(((u < n_prefix) ? ws_v : v_cur) + off + vlo, vd + i * 1024);
      }
    }
  };

  // Per-lane LDS offsets within a tile, fixed for the whole loop, so that the
  // buffer, the sub-step and the key block enter the reads as immediates.
  //  K operand, MFMA kk: key 16 kb + n, chunk 4kk + j (d = 32kk + 8j + [0, 8)).
  //  V operand, block nb: key 4j + (n >> 2) (+32st, +16 for the second read),
  //  columns 16nb + 4(n & 3) .. +3 (chunk 2nb + ((n & 3) >> 1), half n & 1).
  int kofs[4], vofs[8];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) kofs[kk] = chunk_at(n, 4 * kk + j);
  {
    const int ka = 4 * j + (n >> 2);
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) vofs[nb] = vchunk_at(ka, 2 * nb + ((n & 3) >> 1)) + ((n & 1) << 3);
  }

  // One 64-key tile.  MODE 0: softmax against the fixed per-row reference
  // m_run (no rescale); MODE 1: the same, with m_run set from the first
  // sub-step's row maximum (the first tile); MODE 2: lazy running maximum
  // (O and l rescaled when a sub-step's maximum passes m_run + 8).
  auto tile_body = [&](auto bufc, auto modec, int tile) {
    constexpr int buf = decltype(bufc)::value;
    constexpr int MODE = decltype(modec)::value;
    const int u0 = tile * kTileKeys;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of tile `tile` have landed (vmcnt 0)
    __syncthreads();                // every wave's have; the other buffer is free
    if (tile + 1 < n_tiles) fetch(std::integral_constant<int, buf ^ 1>{}, u0 + kTileKeys);
    const uint8_t* kt = buf == 0 ? k_lds0 : k_lds1;
    const uint8_t* vt = buf == 0 ? v_lds0 : v_lds1;

    const bool tile_mask = (u0 + kTileKeys - 1 > diag) || (u0 + kTileKeys > n_keys);
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      // ---- S^T = K * Q^T for keys u0 + 32st + [0, 32), every query-row block
      f32x4 s[2][kRowBlocks];
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
        for (int cb = 0; cb < kRowBlocks; ++cb) s[kb2][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          // key (2st + kb2) * 16 + n: (key & 15) == n, so the swizzle is in kofs
          const bf16x8 a = u4_as_bf16x8(*reinterpret_cast<const uint4*>(kt + kofs[kk] + (2 * st + kb2) * 16 * kRowBytes));
#pragma unroll
          for (int cb = 0; cb < kRowBlocks; ++cb) s[kb2][cb] = mfma16x16x32(a, qb[cb][kk], s[kb2][cb]);
        }
      }

      // ---- online softmax per query row (column n of each block) on raw
      //      scores; the scale enters through one FMA per element.  Lane
      //      (n, j) holds keys 32st + 4j + i (slot i) and 32st + 16 + 4j + i.
      // The P*V operands of this sub-step are read now, so that their LDS
      // latency passes under the softmax below.  B operand of lane (n, j):
      // V[key][16nb + n] for keys 32st + 4j + [0,4) (slots 0..3) and
      // 32st + 16 + 4j + [0,4) (slots 4..7), by two transposing reads: source
      // lane s = n of group j names key +(s >> 2), columns 16nb + 4(s & 3) .. +3.
      bf16x8 bvs[8];
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const uint2 b0 = ds_read_tr16(vt + vofs[nb] + 32 * st * kRowBytes);
        const uint2 b1 = ds_read_tr16(vt + vofs[nb] + (32 * st + 16) * kRowBytes);
        bvs[nb] = u4_as_bf16x8(make_uint4(b0.x, b0.y, b1.x, b1.y));
      }
      const bool need_mask = tile_mask && (u0 + 32 * st + 31 > diag || u0 + 32 * st + 32 > n_keys);
      bf16x8 pa[kRowBlocks];
      if constexpr (MODE == 0) {
        // Masks of both row blocks first, then straight-line code: a row
        // block's exponentials and P*V MFMAs, then the next's (2 % faster
        // than masking and exponentiating each block between branches).
        float sc[kRowBlocks][8];
#pragma unroll
        for (int cb = 0; cb < kRowBlocks; ++cb)
#pragma unroll
          for (int e = 0; e < 8; ++e) sc[cb][e] = s[e >> 2][cb][e & 3];
        if (need_mask) {
#pragma unroll
          for (int cb = 0; cb < kRowBlocks; ++cb) {
            // slot e holds key u0 + 32st + 4j + (e & 3) + 16 (e >> 2); it is
            // visible when that is at most the row's last visible key
            const int rel = min(n_prefix + row_tok[cb], n_keys - 1) - (u0 + 32 * st) - 4 * j;
#pragma unroll
            for (int e = 0; e < 8; ++e) sc[cb][e] = ((e & 3) + 16 * (e >> 2) <= rel) ? sc[cb][e] : -INFINITY;
          }
        }
#pragma unroll
        for (int cb = 0; cb < kRowBlocks; ++cb) {
          const float neg_m = -m_run[cb];
          float p[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(sc[cb][e], qk_scale_log2, neg_m));
          pa[cb] = u4_as_bf16x8(make_uint4(f32x2_to_bf16x2(p[0], p[1]), f32x2_to_bf16x2(p[2], p[3]),
                                           f32x2_to_bf16x2(p[4], p[5]), f32x2_to_bf16x2(p[6], p[7])));
          lsum[cb] = mfma16x16x32(pa[cb], ones, lsum[cb]);
#pragma unroll
          for (int nb = 0; nb < 8; ++nb) o[cb][nb] = mfma16x16x32(pa[cb], bvs[nb], o[cb][nb]);
        }
      } else {
#pragma unroll
        for (int cb = 0; cb < kRowBlocks; ++cb) {
          float sc[8] = {s[0][cb][0], s[0][cb][1], s[0][cb][2], s[0][cb][3],
                         s[1][cb][0], s[1][cb][1], s[1][cb][2], s[1][cb][3]};
          if (need_mask) {
            // slot e holds key u0 + 32st + 4j + (e & 3) + 16 (e >> 2); it is
            // visible when that is at most the row's last visible key
            const int rel = min(n_prefix + row_tok[cb], n_keys - 1) - (u0 + 32 * st) - 4 * j;
#pragma unroll
            for (int e = 0; e < 8; ++e) sc[e] = ((e & 3) + 16 * (e >> 2) <= rel) ? sc[e] : -INFINITY;
          }
          if (MODE == 2 || (MODE == 1 && st == 0)) {
            float tmax = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])), fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
            tmax = max_over_row_groups(tmax);
            tmax *= qk_scale_log2;  // the scale is positive: max commutes with it
            if (MODE == 1) {
              // Key 0 is in this sub-step and every row sees it: finite.
              m_run[cb] = tmax;
            } else if (__any(tmax > m_run[cb] + kLazyMaxSlack)) {
              // Lazy maximum.  The first sub-step holds key 0, which every row
              // sees, so m_run is finite from then on.  A sub-step whose keys
              // are all masked for a row has tmax = -inf and p = 0.
              const float m_new = fmaxf(m_run[cb], tmax);
              const float alpha = __builtin_amdgcn_exp2f(m_run[cb] - m_new);  // 0 on the first sub-step
              m_run[cb] = m_new;
              float ai[4];
#pragma unroll
              for (int i = 0; i < 4; ++i) ai[i] = __shfl(alpha, 4 * j + i);
#pragma unroll
              for (int i = 0; i < 4; ++i) lsum[cb][i] *= ai[i];
#pragma unroll
              for (int nb = 0; nb < 8; ++nb)
#pragma unroll
                for (int i = 0; i < 4; ++i) o[cb][nb][i] *= ai[i];
            }
          }
          const float neg_m = -m_run[cb];
          float p[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(sc[e], qk_scale_log2, neg_m));
          pa[cb] = u4_as_bf16x8(make_uint4(f32x2_to_bf16x2(p[0], p[1]), f32x2_to_bf16x2(p[2], p[3]),
                                           f32x2_to_bf16x2(p[4], p[5]), f32x2_to_bf16x2(p[6], p[7])));
          lsum[cb] = mfma16x16x32(pa[cb], ones, lsum[cb]);
        }
        // ---- O += P * V with the operands read above.
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
#pragma unroll
          for (int cb = 0; cb < kRowBlocks; ++cb) o[cb][nb] = mfma16x16x32(pa[cb], bvs[nb], o[cb][nb]);
        }
      }
    }
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;

  // Fixed reference: m_run is the maximum of each row's first 32 keys, and
  // no later key rescales anything, so the accumulators see only the MFMAs.
  fetch(B0{}, 0);
  tile_body(B0{}, std::integral_constant<int, 1>{}, 0);
  for (int tile = 1; tile < n_tiles; tile += 2) {
    tile_body(B1{}, B0{}, tile);
    if (tile + 1 < n_tiles) tile_body(B0{}, B0{}, tile + 1);
  }
  // A later key can exceed the reference by enough that some p (<= l) or a
  // partial sum of O overflows; non-finite results are kept as such (inf
  // absorbs), so finite l and O mean that nothing overflowed and the result
  // is as exact as with a running maximum.  Otherwise the workgroup runs the
  // tiles again with the lazy running maximum.
  uint32_t worst = 0;
#pragma unroll
  for (int cb = 0; cb < kRowBlocks; ++cb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      worst = max(worst, __float_as_uint(lsum[cb][i]) & 0x7fffffffu);
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) worst = max(worst, __float_as_uint(o[cb][nb][i]) & 0x7fffffffu);
    }
  }
  // (The bits stay out of the compiler's sight: folded into a floating-point
  // class test, the NaN case could be dropped -- the build assumes no NaN
  // operands -- and inf * 0 in the MFMAs makes NaN from an overflow.)
  asm volatile("" : "+v"(worst));
  if (__syncthreads_or(worst >= 0x7f800000u)) {
#pragma unroll
    for (int mb = 0; mb < kRowBlocks; ++mb) {
      m_run[mb] = -INFINITY;
      lsum[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) o[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    fetch(B0{}, 0);
    for (int tile = 0; tile < n_tiles; tile += 2) {
      tile_body(B0{}, std::integral_constant<int, 2>{}, tile);
      if (tile + 1 < n_tiles) tile_body(B1{}, std::integral_constant<int, 2>{}, tile + 1);
    }
  }

  // ---- normalize and store: lane (n, j) holds rows 4j+i of block cb, d = 16nb + n
#pragma unroll
  for (int cb = 0; cb < kRowBlocks; ++cb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rho = (wave * kRowBlocks + cb) * 16 + 4 * j + i;
      const int tok = i0 + rho / G;
      const int head = h0 + rho % G;
      if (tok < n_tokens) {
        const float inv = 1.0f / lsum[cb][i];
        uint16_t* dst = out + ((int64_t)tok * n_q_heads + head) * kHeadDim + n;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          const __bf16 hv = (__bf16)(o[cb][nb][i] * inv);
          dst[16 * nb] = __builtin_bit_cast(uint16_t, hv);
        }
      }
    }
  }
}

template <int G>
hipError_t launch_g(const uint16_t* q, const uint16_t* ws_k, const uint16_t* ws_v, const uint16_t* k_cur,
                    const uint16_t* v_cur, int32_t n_prefix, int32_t n_tokens, int32_t n_q_heads,
                    int32_t n_kv_heads, float qk_scale_log2, uint16_t* out, hipStream_t stream) {
  constexpr int BQ = kRowsPerWg / G;
  dim3 grid((unsigned)((n_tokens + BQ - 1) / BQ), (unsigned)n_kv_heads);
  hipLaunchKernelGGL(prefill_attn_kernel<G>, grid, dim3(kBlock), 0, stream, q, ws_k, ws_v, k_cur, v_cur, n_prefix,
                     n_tokens, n_q_heads, n_kv_heads, qk_scale_log2, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_attention(const uint16_t* q, const uint16_t* ws_k, const uint16_t* ws_v,
                                    const uint16_t* k_cur, const uint16_t* v_cur, int32_t n_prefix,
                                    int32_t n_tokens, int32_t n_q_heads, int32_t n_kv_heads, float sm_scale,
                                    uint16_t* out, hipStream_t stream) {
  const float qk_scale_log2 = sm_scale * 1.4426950408889634f;
  switch (n_q_heads / n_kv_heads) {
    case 1: return launch_g<1>(q, ws_k, ws_v, k_cur, v_cur, n_prefix, n_tokens, n_q_heads, n_kv_heads, qk_scale_log2, out, stream);
    case 2: return launch_g<2>(q, ws_k, ws_v, k_cur, v_cur, n_prefix, n_tokens, n_q_heads, n_kv_heads, qk_scale_log2, out, stream);
    case 4: return launch_g<4>(q, ws_k, ws_v, k_cur, v_cur, n_prefix, n_tokens, n_q_heads, n_kv_heads, qk_scale_log2, out, stream);
    case 8: return launch_g<8>(q, ws_k, ws_v, k_cur, v_cur, n_prefix, n_tokens, n_q_heads, n_kv_heads, qk_scale_log2, out, stream);
    case 16: return launch_g<16>(q, ws_k, ws_v, k_cur, v_cur, n_prefix, n_tokens, n_q_heads, n_kv_heads, qk_scale_log2, out, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fp8kv
