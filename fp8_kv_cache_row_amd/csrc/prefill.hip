// prefill.hip -- causal chunked-prefill attention over [bf16 workspace prefix ;
// bf16 current chunk] on the gfx950 bf16 MFMA.
//
// FreeToken PR #853 "opt-in FP8 KV cache", "What changes": historical FP8 rows
// are reconstructed once per layer into one shared BF16 workspace and the
// current chunk's K/V stay BF16; "Paired end-to-end A/B": the 8K
// historical-prefix + 8K new-token operator.
//
// Work decomposition: a workgroup owns 128 "query rows", each one
// (query token, query head) pair of a single KV head's group (128/G tokens x
// G heads), so one K/V tile staged in LDS feeds every query head of the
// group.  Four waves take 32 rows each.  Per 64-key tile a wave computes
// S^T = K * Q^T (keys on MFMA rows, query rows on columns) so that a lane holds
// 16 keys of one query row: the row max/sum need two cross-lane steps, and the
// same registers are the k-slots of the P*V MFMA.  V is stored transposed in
// LDS ([d][key]) so the P*V operand is a plain 8-byte LDS read.
//
// Pipelining: K/V tiles are double-buffered in LDS.  The global loads of tile
// t+1 are issued into registers before tile t is computed and written to the
// other buffer afterwards, so one barrier per tile suffices and the load
// latency hides behind the MFMA work.  A tile is computed as two 32-key
// sub-steps (QK^T, softmax, P*V each) to keep the live registers low.  Online
// softmax in log2 units with a lazy maximum (O and l are rescaled only when a
// sub-step's maximum exceeds the running one by more than 8), so the
// accumulators are normally touched by the MFMA alone.  Workgroups with the most keys (the last query tokens) are
// launched first.
#include <math.h>

#include "fp8kv_device.h"

namespace fp8kv {

namespace {

constexpr int kBlock = 256;
constexpr int kRowsPerWg = 128;
constexpr int kTileKeys = 64;
// K tile: [64 keys][16 chunks of 16 B]; chunk c of key m is stored at chunk
// position c ^ (m & 15) so that 16 lanes reading one chunk of 16 keys hit all
// 64 banks.
constexpr int kKRowBytes = kHeadDim * 2;
constexpr int kKTileBytes = kTileKeys * kKRowBytes;
// V^T tile: [128 d][16 chunks of 8 B (4 keys)]; chunk q of row d is stored at
// position q ^ vswz(d).  vswz takes 16 distinct values both over d = 16b + n
// (n = 0..15: the rows one P*V operand read touches) and over d = 8c + k
// (c = 0..15: the rows one transposing store touches), so neither side has
// bank conflicts.
constexpr int kVRowBytes = kTileKeys * 2;
__device__ __forceinline__ int vswz(int d) { return (d ^ (d >> 3)) & 15; }
constexpr int kVTileBytes = kHeadDim * kVRowBytes;
constexpr float kLazyMaxSlack = 8.0f;

// One thread's share of a K/V tile in registers: 4 K chunks (16 B each) and
// 4 keys x 8 d of V.
struct TileRegs {
  uint4 k[4];
  uint4 v[4];
};

// Fast path: the whole tile lies in the workspace or in the chunk (below
// n_keys), so every element address is one tile base plus a per-thread offset
// fixed for the whole loop.
__device__ __forceinline__ void load_tile_run(TileRegs& r, const uint16_t* __restrict__ kbase,
                                              const uint16_t* __restrict__ vbase, const int (&kofs)[4],
                                              const int (&vofs)[4]) {
#pragma unroll
  for (int it = 0; it < 4; ++it) r.k[it] = *reinterpret_cast<const uint4*>(kbase + kofs[it]);
#pragma unroll
  for (int e = 0; e < 4; ++e) r.v[e] = *reinterpret_cast<const uint4*>(vbase + vofs[e]);
}

// General path (a tile that straddles the workspace/chunk boundary or the
// last visible key).
__device__ __forceinline__ void load_tile(TileRegs& r, const uint16_t* __restrict__ ws_k,
                                          const uint16_t* __restrict__ ws_v, const uint16_t* __restrict__ k_cur,
                                          const uint16_t* __restrict__ v_cur, int n_prefix, int n_keys, int u0,
                                          int64_t kv_row, int g, int tid) {
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int c = tid + kBlock * it;
    const int u = u0 + (c >> 4), ch = c & 15;
    // keys past n_keys re-read the last valid key (never weighted: masked)
    const int uc = min(u, n_keys - 1);
    const uint16_t* src = (uc < n_prefix) ? ws_k + (int64_t)uc * kv_row : k_cur + (int64_t)(uc - n_prefix) * kv_row;
    r.k[it] = *reinterpret_cast<const uint4*>(src + (int64_t)g * kHeadDim + ch * 8);
  }
  const int kg = tid >> 4, c = tid & 15;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int uc = min(u0 + 4 * kg + e, n_keys - 1);
    const uint16_t* src = (uc < n_prefix) ? ws_v + (int64_t)uc * kv_row : v_cur + (int64_t)(uc - n_prefix) * kv_row;
    r.v[e] = *reinterpret_cast<const uint4*>(src + (int64_t)g * kHeadDim + c * 8);
  }
}

__device__ __forceinline__ void store_tile(const TileRegs& r, uint8_t* k_lds, uint8_t* v_lds, int tid) {
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int c = tid + kBlock * it;
    const int key = c >> 4, ch = c & 15;
    *reinterpret_cast<uint4*>(k_lds + key * kKRowBytes + ((ch ^ (key & 15)) << 4)) = r.k[it];
  }
  // V^T: this thread's 4 keys (4kg..4kg+3) at d = 8c..8c+7 -> 8 rows of 8 bytes
  const int kg = tid >> 4, c = tid & 15;
  const uint32_t w[4][4] = {{r.v[0].x, r.v[0].y, r.v[0].z, r.v[0].w},
                            {r.v[1].x, r.v[1].y, r.v[1].z, r.v[1].w},
                            {r.v[2].x, r.v[2].y, r.v[2].z, r.v[2].w},
                            {r.v[3].x, r.v[3].y, r.v[3].z, r.v[3].w}};
#pragma unroll
  for (int p = 0; p < 4; ++p) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const uint32_t sel = s ? 0x07060302u : 0x05040100u;
      const uint32_t lo = __builtin_amdgcn_perm(w[1][p], w[0][p], sel);  // keys 0,1
      const uint32_t hi = __builtin_amdgcn_perm(w[3][p], w[2][p], sel);  // keys 2,3
      const int d = 8 * c + 2 * p + s;
      *reinterpret_cast<uint2*>(v_lds + d * kVRowBytes + ((kg ^ vswz(d)) << 3)) = make_uint2(lo, hi);
    }
  }
}

template <int G>
__global__ __launch_bounds__(kBlock) void prefill_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ ws_k, const uint16_t* __restrict__ ws_v,
    const uint16_t* __restrict__ k_cur, const uint16_t* __restrict__ v_cur, int32_t n_prefix, int32_t n_tokens,
    int32_t n_q_heads, int32_t n_kv_heads, float qk_scale_log2, uint16_t* __restrict__ out) {
  constexpr int BQ = kRowsPerWg / G;  // query tokens per workgroup
  __shared__ __attribute__((aligned(16))) uint8_t k_lds[2][kKTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t v_lds[2][kVTileBytes];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int n = lane & 15;
  const int j = lane >> 4;
  const int g = blockIdx.y;
  const int h0 = g * G;
  const int i0 = (gridDim.x - 1 - blockIdx.x) * BQ;  // most keys first
  const int i_last = min(i0 + BQ, n_tokens) - 1;
  const int n_keys = n_prefix + i_last + 1;  // keys any row of this workgroup may see

  // Q^T operand for the wave's two 16-row column blocks; rows past the chunk
  // reuse the last token (never stored).
  bf16x8 qb[2][4];
  int row_tok[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int rho = wave * 32 + cb * 16 + n;
    const int tok = min(i0 + rho / G, n_tokens - 1);
    const int head = h0 + rho % G;
    row_tok[cb] = tok;
    const uint16_t* qp = q + ((int64_t)tok * n_q_heads + head) * kHeadDim + 8 * j;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qb[cb][kk] = u4_as_bf16x8(*reinterpret_cast<const uint4*>(qp + 32 * kk));
  }

  float m_run[2] = {-INFINITY, -INFINITY};  // lazy running max of row n (log2 units)
  float l_part[2] = {0.f, 0.f};             // this lane's share of the row sum
  f32x4 o[2][8];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) o[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int64_t kv_row = (int64_t)n_kv_heads * kHeadDim;  // elements between tokens
  const int n_tiles = (n_keys + kTileKeys - 1) / kTileKeys;
  // first key index at which any row of this workgroup needs the causal mask
  const int diag = n_prefix + i0;

  // Per-thread element offsets of its tile share, relative to the tile's first key.
  int kofs[4], vofs[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) kofs[it] = ((tid >> 4) + 16 * it) * (int)kv_row + g * kHeadDim + (tid & 15) * 8;
#pragma unroll
  for (int e = 0; e < 4; ++e) vofs[e] = (4 * (tid >> 4) + e) * (int)kv_row + g * kHeadDim + (tid & 15) * 8;
  auto fetch = [&](TileRegs& r, int u0) {
    if (u0 + kTileKeys <= n_prefix) {
      load_tile_run(r, ws_k + (int64_t)u0 * kv_row, ws_v + (int64_t)u0 * kv_row, kofs, vofs);
    } else if (u0 >= n_prefix && u0 + kTileKeys <= n_keys) {
      load_tile_run(r, k_cur + (int64_t)(u0 - n_prefix) * kv_row, v_cur + (int64_t)(u0 - n_prefix) * kv_row, kofs,
                    vofs);
    } else {
      load_tile(r, ws_k, ws_v, k_cur, v_cur, n_prefix, n_keys, u0, kv_row, g, tid);
    }
  };

  TileRegs regs;
  fetch(regs, 0);
  store_tile(regs, k_lds[0], v_lds[0], tid);

  for (int tile = 0; tile < n_tiles; ++tile) {
    const int u0 = tile * kTileKeys;
    const int buf = tile & 1;
    __syncthreads();  // tile `tile` is in buf; everyone is done with the other buffer
    const bool more = tile + 1 < n_tiles;
    if (more) fetch(regs, u0 + kTileKeys);
    const uint8_t* kt = k_lds[buf];
    const uint8_t* vt = v_lds[buf];

    // Two 32-key sub-steps per tile: S^T for key blocks 2st, 2st+1, softmax,
    // then P*V; live score/operand registers stay at one sub-step's worth.
    const bool tile_mask = (u0 + kTileKeys - 1 > diag) || (u0 + kTileKeys > n_keys);
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      // ---- S^T = K * Q^T for keys u0 + 32st + [0, 32), both query-row blocks
      f32x4 s[2][2];
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        s[kb2][0] = f32x4{0.f, 0.f, 0.f, 0.f};
        s[kb2][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int key = (2 * st + kb2) * 16 + n;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int ch = 4 * kk + j;  // d = 32kk + 8j + [0, 8)
          const bf16x8 a = u4_as_bf16x8(*reinterpret_cast<const uint4*>(kt + key * kKRowBytes + ((ch ^ (key & 15)) << 4)));
          s[kb2][0] = mfma16x16x32(a, qb[0][kk], s[kb2][0]);
          s[kb2][1] = mfma16x16x32(a, qb[1][kk], s[kb2][1]);
        }
      }

      // ---- online softmax per query row (column n of each block) on raw
      //      scores; the scale enters through one FMA per element.  Lane
      //      (n, j) holds keys 32st + 4j + i (slot i) and 32st + 16 + 4j + i.
      const bool need_mask = tile_mask && (u0 + 32 * st + 31 > diag || u0 + 32 * st + 32 > n_keys);
      bf16x8 pa[2];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        float sc[8] = {s[0][cb][0], s[0][cb][1], s[0][cb][2], s[0][cb][3],
                       s[1][cb][0], s[1][cb][1], s[1][cb][2], s[1][cb][3]};
        if (need_mask) {
          const int limit = min(n_prefix + row_tok[cb], n_keys - 1);  // last visible key of this row
#pragma unroll
          for (int e = 0; e < 8; ++e)
            sc[e] = (u0 + 32 * st + 16 * (e >> 2) + 4 * j + (e & 3) <= limit) ? sc[e] : -INFINITY;
        }
        float tmax = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])), fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
        tmax = max_over_row_groups(tmax);
        tmax *= qk_scale_log2;  // the scale is positive: max commutes with it
        // Lazy maximum.  The first sub-step holds key 0, which every row
        // sees, so m_run is finite from then on.  A sub-step whose keys are
        // all masked for a row has tmax = -inf and p = 0.
        if (__any(tmax > m_run[cb] + kLazyMaxSlack)) {
          const float m_new = fmaxf(m_run[cb], tmax);
          const float alpha = __builtin_amdgcn_exp2f(m_run[cb] - m_new);  // 0 on the first sub-step
          m_run[cb] = m_new;
          l_part[cb] *= alpha;
          float ai[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) ai[i] = __shfl(alpha, 4 * j + i);
#pragma unroll
          for (int nb = 0; nb < 8; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i) o[cb][nb][i] *= ai[i];
        }
        const float neg_m = -m_run[cb];
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(sc[e], qk_scale_log2, neg_m));
        l_part[cb] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
        pa[cb] = u4_as_bf16x8(make_uint4(f32x2_to_bf16x2(p[0], p[1]), f32x2_to_bf16x2(p[2], p[3]),
                                         f32x2_to_bf16x2(p[4], p[5]), f32x2_to_bf16x2(p[6], p[7])));
      }

      // ---- O += P * V: B operand = V^T rows d = 16nb + n, the lane's 8 keys
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const int d = 16 * nb + n;
        const int q0 = 8 * st + j;      // keys 32st + 4j .. +3
        const int q1 = 8 * st + 4 + j;  // keys 32st + 16 + 4j .. +3
        const uint8_t* rowp = vt + d * kVRowBytes;
        const uint2 b0 = *reinterpret_cast<const uint2*>(rowp + ((q0 ^ vswz(d)) << 3));
        const uint2 b1 = *reinterpret_cast<const uint2*>(rowp + ((q1 ^ vswz(d)) << 3));
        const bf16x8 bv = u4_as_bf16x8(make_uint4(b0.x, b0.y, b1.x, b1.y));
        o[0][nb] = mfma16x16x32(pa[0], bv, o[0][nb]);
        o[1][nb] = mfma16x16x32(pa[1], bv, o[1][nb]);
      }
    }

    // ---- the next tile into the other buffer (its last readers finished
    //      before this iteration's barrier)
    if (more) store_tile(regs, k_lds[buf ^ 1], v_lds[buf ^ 1], tid);
  }

  // ---- normalize and store: lane (n, j) holds rows 4j+i of block cb, d = 16nb + n
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    float l_tot = l_part[cb] + __shfl_xor(l_part[cb], 16);
    l_tot += __shfl_xor(l_tot, 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float li = __shfl(l_tot, 4 * j + i);
      const int rho = wave * 32 + cb * 16 + 4 * j + i;
      const int tok = i0 + rho / G;
      const int head = h0 + rho % G;
      if (tok < n_tokens) {
        const float inv = 1.0f / li;
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
