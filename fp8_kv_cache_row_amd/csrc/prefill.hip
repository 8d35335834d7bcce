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
// V^T tile: [128 d][16 chunks of 8 B (4 keys)]; chunk q of row d is stored at
// position q ^ ((d >> 1) & 7).
constexpr int kVRowBytes = kTileKeys * 2;


template <int G>
__global__ __launch_bounds__(kBlock) void prefill_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ ws_k, const uint16_t* __restrict__ ws_v,
    const uint16_t* __restrict__ k_cur, const uint16_t* __restrict__ v_cur, int32_t n_prefix, int32_t n_tokens,
    int32_t n_q_heads, int32_t n_kv_heads, float qk_scale_log2, uint16_t* __restrict__ out) {
  constexpr int BQ = kRowsPerWg / G;  // query tokens per workgroup
  __shared__ __attribute__((aligned(16))) uint8_t k_lds[kTileKeys * kKRowBytes];
  __shared__ __attribute__((aligned(16))) uint8_t v_lds[kHeadDim * kVRowBytes];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int n = lane & 15;
  const int j = lane >> 4;
  const int g = blockIdx.y;
  const int h0 = g * G;
  const int i0 = blockIdx.x * BQ;
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

  float m_run[2] = {-INFINITY, -INFINITY};
  float l_part[2] = {0.f, 0.f};
  f32x4 o[2][8];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) o[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int64_t kv_row = (int64_t)n_kv_heads * kHeadDim;  // elements between tokens
  const int n_tiles = (n_keys + kTileKeys - 1) / kTileKeys;
  // first key index at which any row of this workgroup needs the causal mask
  const int diag = n_prefix + i0;

  for (int tile = 0; tile < n_tiles; ++tile) {
    const int u0 = tile * kTileKeys;
    __syncthreads();  // previous tile fully consumed
    // ---- stage K tile: 1024 chunks of 16 B, 4 per thread
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int c = tid + kBlock * it;
      const int key = c >> 4, ch = c & 15;
      const int u = u0 + key;
      uint4 val = make_uint4(0u, 0u, 0u, 0u);
      if (u < n_keys) {
        const uint16_t* src = (u < n_prefix) ? ws_k + (int64_t)u * kv_row : k_cur + (int64_t)(u - n_prefix) * kv_row;
        val = *reinterpret_cast<const uint4*>(src + (int64_t)g * kHeadDim + ch * 8);
      }
      *reinterpret_cast<uint4*>(k_lds + key * kKRowBytes + ((ch ^ (key & 15)) << 4)) = val;
    }
    // ---- stage V^T tile: thread loads keys 4kg..4kg+3 at d-chunk c (8 d)
    {
      const int kg = tid >> 4, c = tid & 15;
      uint4 r4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int u = u0 + 4 * kg + e;
        r4[e] = make_uint4(0u, 0u, 0u, 0u);
        if (u < n_keys) {
          const uint16_t* src = (u < n_prefix) ? ws_v + (int64_t)u * kv_row : v_cur + (int64_t)(u - n_prefix) * kv_row;
          r4[e] = *reinterpret_cast<const uint4*>(src + (int64_t)g * kHeadDim + c * 8);
        }
      }
      const uint32_t w[4][4] = {{r4[0].x, r4[0].y, r4[0].z, r4[0].w},
                                {r4[1].x, r4[1].y, r4[1].z, r4[1].w},
                                {r4[2].x, r4[2].y, r4[2].z, r4[2].w},
                                {r4[3].x, r4[3].y, r4[3].z, r4[3].w}};
#pragma unroll
      for (int p = 0; p < 4; ++p) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const uint32_t sel = s ? 0x07060302u : 0x05040100u;
          const uint32_t lo = __builtin_amdgcn_perm(w[1][p], w[0][p], sel);  // keys 0,1
          const uint32_t hi = __builtin_amdgcn_perm(w[3][p], w[2][p], sel);  // keys 2,3
          const int d = 8 * c + 2 * p + s;
          *reinterpret_cast<uint2*>(v_lds + d * kVRowBytes + ((kg ^ ((d >> 1) & 7)) << 3)) = make_uint2(lo, hi);
        }
      }
    }
    __syncthreads();

    // ---- S^T = K * Q^T: 4 key blocks x 2 query-row blocks
    f32x4 s[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb][0] = f32x4{0.f, 0.f, 0.f, 0.f};
      s[kb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int key = kb * 16 + n;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int ch = 4 * kk + j;  // d = 32kk + 8j + [0, 8)
        const bf16x8 a = u4_as_bf16x8(*reinterpret_cast<const uint4*>(k_lds + key * kKRowBytes + ((ch ^ (key & 15)) << 4)));
        s[kb][0] = mfma16x16x32(a, qb[0][kk], s[kb][0]);
        s[kb][1] = mfma16x16x32(a, qb[1][kk], s[kb][1]);
      }
    }

    // ---- online softmax per query row (column n of each block)
    const bool need_mask = (u0 + kTileKeys - 1 > diag) || (u0 + kTileKeys > n_keys);
    bf16x8 pa[2][2];  // [row block][k-step]
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int limit = n_prefix + row_tok[cb];  // last visible key for this row
      float sc[16];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = s[kb][cb][i] * qk_scale_log2;
          if (need_mask) {
            const int u = u0 + kb * 16 + 4 * j + i;
            v = (u <= limit) ? v : -INFINITY;
          }
          sc[kb * 4 + i] = v;
        }
      }
      float tmax = sc[0];
#pragma unroll
      for (int e = 1; e < 16; ++e) tmax = fmaxf(tmax, sc[e]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float m_new = fmaxf(m_run[cb], tmax);
      // a row whose keys are all masked so far keeps m = -inf and p = 0
      const float alpha = (m_new == -INFINITY) ? 1.0f : exp2f(m_run[cb] - m_new);
      m_run[cb] = m_new;
      float p[16], psum = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        p[e] = (m_new == -INFINITY) ? 0.0f : exp2f(sc[e] - m_new);
        psum += p[e];
      }
      l_part[cb] = l_part[cb] * alpha + psum;
      // k-step st uses key blocks 2st (slots 0..3) and 2st+1 (slots 4..7)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const float* pb0 = p + (2 * st) * 4;
        const float* pb1 = p + (2 * st + 1) * 4;
        uint4 u;
        u.x = f32x2_to_bf16x2(pb0[0], pb0[1]);
        u.y = f32x2_to_bf16x2(pb0[2], pb0[3]);
        u.z = f32x2_to_bf16x2(pb1[0], pb1[1]);
        u.w = f32x2_to_bf16x2(pb1[2], pb1[3]);
        pa[cb][st] = u4_as_bf16x8(u);
      }
      float ai[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ai[i] = __shfl(alpha, 4 * j + i);
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[cb][nb][i] *= ai[i];
    }

    // ---- O += P * V: B operand = V^T rows d = 16nb + n, keys of the lane's k-slots
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const int d = 16 * nb + n;
        const int q0 = 8 * st + j;      // keys 32st + 4j .. +3
        const int q1 = 8 * st + 4 + j;  // keys 32st + 16 + 4j .. +3
        const uint8_t* rowp = v_lds + d * kVRowBytes;
        const uint2 b0 = *reinterpret_cast<const uint2*>(rowp + ((q0 ^ ((d >> 1) & 7)) << 3));
        const uint2 b1 = *reinterpret_cast<const uint2*>(rowp + ((q1 ^ ((d >> 1) & 7)) << 3));
        const bf16x8 bv = u4_as_bf16x8(make_uint4(b0.x, b0.y, b1.x, b1.y));
        o[0][nb] = mfma16x16x32(pa[0][st], bv, o[0][nb]);
        o[1][nb] = mfma16x16x32(pa[1][st], bv, o[1][nb]);
      }
    }
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
