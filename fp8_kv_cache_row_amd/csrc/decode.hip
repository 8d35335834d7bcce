// decode.hip -- split-K GQA decode attention over the page-size-1 FP8 row pool.
//
// FreeToken PR #897 "perf(attention): add packed fp8 kv reads on gfx1201",
// description and "Fresh R9700 stage-1 A/B": a first stage computes one
// partial per (head group, split) over FP8 rows fetched through the row table
// (page size 1, randomized physical slots) and a merge kernel combines the
// partials.  FreeToken PR #853 "What changes": per-row FP32 scales.
//
// gfx950 design (not the pages' RDNA4 kernel), described for the headline
// shape (one query row per request, head dim 128, E4M3 codes); the template
// parameters below generalize it to head dim 256, several query rows per
// request (FreeToken PR #897 description: #900's multi-row decode), a sliding
// key window and INT8 codes ("Regression and CUDA isolation" lists all four):
//  * A workgroup (8 waves) covers one split of one (request, KV head); a wave
//    takes two 32-key steps at a time.  The request length is read with a
//    vector load next to the first (speculative, host-bounded) table read, so
//    it costs no extra round trip, and no code byte past the length's 64-key
//    group is fetched.
//  * Every lane loads exactly the code bytes its MFMA operands need, straight
//    into registers: for keys on the MFMA rows, 16-byte K chunks; for the P*V
//    contraction, D/16 bytes of V per key, 16 lanes covering one whole V row.
//    All loads of a group are in flight before the first wait; only row
//    indices and scales pass through LDS.
//  * QK^T runs on the bf16 MFMA 16x16x32 with E4M3 (or INT8) codes widened
//    exactly to bf16.  S^T = K * Q^T puts keys on the MFMA rows and the
//    columns -- the G query heads of the group, or (query row, head) pairs --
//    on the MFMA columns, so each lane holds 8 keys of one column: the
//    column maximum needs two cross-lane steps, and those 8 keys are exactly
//    the k-slots this lane feeds to the P*V MFMA, so P never moves between
//    lanes.  The per-row K scale and the softmax scale multiply the score tile
//    after the MFMA (one FMA with the reference); the per-row V scale is
//    folded into P.
//  * Softmax in log2 units against a fixed reference per column: the maximum
//    of the column's first visible step.  p = 2^(s - ref) is never rescaled,
//    so after that step there is no maximum and no rescale branch (whose
//    join costs register copies of O) -- 9.7-9.8 against 10.1-10.2 us for
//    the 32K stage 1.  A key far enough above the reference overflows p, l
//    or O into inf or NaN, which then stays; a wave whose l and O are not
//    finite sums its keys again with a lazy running maximum (moved, with O
//    rescaled, only when a step's maximum passes it by more than 8).  At head
//    dim 256 the registers leave no room for the second pass's code and the
//    lazy maximum is the only one.
//  * Waves merge through LDS; one (o, log2-sum-exp) partial per split.
//  * An appending decode step (the new token quantized on write) with one row
//    per request and one workgroup round lets stage 1 take the new token:
//    one wave of split 0's workgroup quantizes it into its pool row while
//    that wave would otherwise wait on the other waves' rows, scores it and
//    folds it into split 0's partial, so the merge is the plain one -- 12.9
//    against 13.2 us for the 32K step with the merge taking the token.
//  * The grid places the KV heads of one split on one XCD, next to each other
//    in dispatch order, so they share that XCD's L2 lines of the table and of
//    the rows' scales; grids of several rounds (batches, long contexts) use
//    512-key splits and a streaming shape of three 4-wave workgroups per CU.

#include <math.h>

#include <type_traits>

#include "fp8kv_device.h"

namespace fp8kv {

// Measurement build only (FP8KV_WAVE_TIMELINE, the benchmark's timeline
// library; the product library is built without it): each wave of stage 1
// records the 100 MHz real-time counter at fixed points -- entry, its first
// group's row indices in, its scales in, its first step done, all steps done,
// partials stored -- in fp8kv_timeline[(workgroup * waves + wave) * 8 + point]
// for the first kTimelineWorkgroups workgroups of a launch.
#ifdef FP8KV_WAVE_TIMELINE
constexpr int kTimelineWorkgroups = 1024;
__device__ unsigned long long fp8kv_timeline[kTimelineWorkgroups * 8 * 8];
#define FP8KV_MARK(point, cond)                                                                           \
  do {                                                                                                   \
    __builtin_amdgcn_sched_barrier(0);                                                                   \
    const unsigned long long t_ = __builtin_amdgcn_s_memrealtime();                                      \
    const int wg_ = (int)(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z));              \
    if ((cond) && lane == 0 && wg_ < kTimelineWorkgroups) fp8kv_timeline[(wg_ * 8 + wave) * 8 + (point)] = t_; \
    __builtin_amdgcn_sched_barrier(0);                                                                   \
  } while (0)
#else
#define FP8KV_MARK(point, cond) \
  do {                          \
  } while (0)
#endif

namespace {

constexpr float kLazyMaxSlack = 8.0f;  // log2 units: p <= 2^8 between rescales
constexpr float kLog2e = 1.4426950408889634f;
// Running maximum before any visible key: finite, so a column with no visible
// key in a step gets p = exp2(-inf - kNoMax) = 0 instead of NaN, and far below
// every real score.
constexpr float kNoMax = -1.0e30f;

// Key order inside a 32-key step: k-group j of the P*V contraction holds keys
// 4j..4j+3 (first 16-key MFMA block) and 16+4j..16+4j+3 (second block).
__device__ __forceinline__ int step_key(int j, int r) { return (r < 4) ? 4 * j + r : 12 + 4 * j + r; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// E consecutive values per lane: bf16 bit patterns in E/2 dwords, fp32 in a vector.
template <int E>
struct LaneVec {
  typedef float F __attribute__((ext_vector_type(E)));
  typedef uint32_t U __attribute__((ext_vector_type(E / 2)));
};

// One new token's K and V rows of a KV head, spread over a wave (lane l holds
// d = E*l .. E*l + E-1 as bf16 pairs), quantized exactly as the
// quantize-on-write kernel does it (the same codec functions and a wave-wide
// amax): the codes (byte e of kc / vc is element e), the fp32 scales, and the
// values the codes decode to (before the scale).
template <int E>
struct NewTokenCodes {
  uint32_t kc, vc;
  float sk, sv;
  float kd[4], vd[4];
};
template <int E, int F>
__device__ __forceinline__ NewTokenCodes<E> quantize_new_token(typename LaneVec<E>::U k2, typename LaneVec<E>::U v2) {
  using Code = Codec<F>;
  NewTokenCodes<E> r;
  float kx[E], vx[E];
#pragma unroll
  for (int e = 0; e < E; e += 2) {
    kx[e] = bf16lo_to_f32(k2[e / 2]);
    kx[e + 1] = bf16hi_to_f32(k2[e / 2]);
    vx[e] = bf16lo_to_f32(v2[e / 2]);
    vx[e + 1] = bf16hi_to_f32(v2[e / 2]);
  }
  float ka = 0.f, va = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    ka = fmaxf(ka, fabsf(kx[e]));
    va = fmaxf(va, fabsf(vx[e]));
  }
  ka = wave_max(ka);
  va = wave_max(va);
  r.sk = Code::scale(ka);
  r.sv = Code::scale(va);
  r.kc = Code::template pack2<false>(Code::prescale(kx[0], ka, r.sk), Code::prescale(kx[1], ka, r.sk), 0u);
  r.vc = Code::template pack2<false>(Code::prescale(vx[0], va, r.sv), Code::prescale(vx[1], va, r.sv), 0u);
  if constexpr (E == 4) {
    r.kc = Code::template pack2<true>(Code::prescale(kx[2], ka, r.sk), Code::prescale(kx[3], ka, r.sk), r.kc);
    r.vc = Code::template pack2<true>(Code::prescale(vx[2], va, r.sv), Code::prescale(vx[3], va, r.sv), r.vc);
  }
  Code::widen4(r.kc, r.kd);
  Code::widen4(r.vc, r.vd);
  return r;
}

// The new token of a single-row appending call when stage 1 takes it
// (k_new null: it does not): bf16 K/V rows [B][new_token_stride], head g at
// g * D, quantized into pool row new_slots[b].
struct FoldKernelArgs {
  const uint16_t* k_new;
  const uint16_t* v_new;
  int64_t new_token_stride;
  const int32_t* new_slots;
};

// Compile-time shape of one stage-1 instantiation.
//   D       head dim (128 or 256).
//   NT      16-wide column tiles per workgroup.  A column is one (query row i,
//           query head hh of the group) pair, c = i * G + hh.
//   MULTI   several query rows per request (columns c >= G exist); otherwise
//           the columns are the G heads of one row and G is a template value.
//   WINDOW  a sliding key window: the key range starts at the first row's
//           lowest visible position, so the table read waits for the length.
//   F       the code format (E4M3FN or INT8), widened exactly to bf16.
//   STREAM  4-wave workgroups, three per compute unit (at most 168
//           registers), for grids of several rounds.
template <int G_, int D_, int NT_, bool MULTI_, bool WINDOW_, int F_, bool STREAM_ = false>
struct Stage1 {
  static constexpr int G = G_, D = D_, NT = NT_, F = F_;
  static constexpr bool MULTI = MULTI_, WINDOW = WINDOW_, STREAM = STREAM_;
  using Code = Codec<F_>;
  // Registers: NT * D / 16 accumulators of 4 floats each, NT * D / 32 query
  // operands and one or two steps of codes in flight.  Wide shapes run 4
  // waves (one per SIMD, 512 registers each) instead of 8.
  // The streaming shape: 4-wave workgroups with two 32-key steps in flight
  // per wave and at most 168 registers, so three workgroups share a compute
  // unit (12 waves, 768 keys in flight per CU against 512 for one 8-wave
  // workgroup of the one-round shape).  Measured on the 16-request batch:
  // 82 us, against 86 us for two 8-wave workgroups of one step per wave.
  static constexpr int kWaves = STREAM ? 4 : ((NT * D >= 512) ? 4 : kDecodeWaves);
  static constexpr int kBlock = kWaves * kWave;
  // 32-key steps loaded at once: two (a whole 512-key split in one group of
  // the 8 waves), except at D = 256 for the several-row tiles and G = 1,
  // whose registers hold one (one row's two steps at D = 256 need all 256,
  // and at G = 1 the compiler spills two).
  static constexpr int kSteps =
      STREAM ? 2 : ((D == 128 || kWaves == 4 || (NT == 1 && !MULTI && G > 1)) ? kDecodeTilesPerWave : 1);
  static constexpr int kWavesPerEU = STREAM ? 3 : 1;  // minimum waves per SIMD the registers allow
  static_assert(!STREAM || (D == 128 && NT == 1 && !MULTI && !WINDOW), "streaming shape: one row, D = 128");
  static constexpr int kGroupKeys = kSteps * kDecodeTileKeys;
  // Row indices and scales are loaded one key per lane; a 32-key group leaves
  // the upper half-wave reading duplicates into padding.
  static constexpr int kRowSlots = (kGroupKeys + kWave - 1) / kWave;
  static constexpr int kKC = D / 64;  // 16-byte K chunks per key and lane
  static constexpr int kQK = D / 32;  // QK^T MFMAs per 16-key block
  static constexpr int kVW = D / 64;  // V dwords per key and lane (D / 16 bytes)
  static constexpr int kNB = D / 16;  // O column blocks: lane column n holds d = kNB * n + nb
  static constexpr int kPassCols = MULTI ? 16 : G;  // LDS columns per epilogue pass
  static_assert(D == 128 || D == 256, "head dim 128 or 256");
  static_assert(G >= 1 && G <= 16, "query heads per KV head must fit one 16-wide MFMA tile");
  static_assert(kGroupKeys % kWave == 0 || kGroupKeys == kWave / 2, "a group covers whole or half waves of row indices");
  static_assert(kSteps >= 1 && kSteps <= 4, "up to four steps in flight per wave");
};

// Code loads, plain or non-temporal (NT: the line is not kept for reuse --
// for a pool whose KV heads never share a line, where it streams the codes
// from HBM faster).
template <bool NT>
__device__ __forceinline__ u32x4 load_code16(const uint8_t* p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  else
    return *reinterpret_cast<const u32x4*>(p);
}

template <int W, bool NT>
__device__ __forceinline__ void load_v_words(const uint8_t* p, uint32_t (&w)[W]) {
  if constexpr (W == 2) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 t = NT ? __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p))
                       : *reinterpret_cast<const u32x2*>(p);
    w[0] = t.x;
    w[1] = t.y;
  } else {
    static_assert(W == 4, "8 or 16 bytes of V per key and lane");
    const u32x4 t = load_code16<NT>(p);
    w[0] = t.x;
    w[1] = t.y;
    w[2] = t.z;
    w[3] = t.w;
  }
}

// Lanes i and i ^ 8 of each 16-lane row exchange a dword: lanes in the banks
// of BANKS (bit b: lanes 4b .. 4b+3 of the row) take src from their partner,
// the others keep old.
template <int BANKS>
__device__ __forceinline__ uint32_t swap8_into(uint32_t old, uint32_t src) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)src, 0x128 /* row_ror:8 */, 0xF, BANKS, false);
}

// NTL: the codes are read with non-temporal loads (a pool whose KV heads never
// share a 128-byte line).  FOLD: the launch also takes each request's new
// token (see kFold below); a separate instantiation, so that the plain stage 1
// keeps its registers and schedule.
template <class C, bool NTL, bool FOLD>
__global__ __launch_bounds__(C::kBlock) __attribute__((amdgpu_waves_per_eu(C::kWavesPerEU))) void decode_stage1_kernel(
    const uint8_t* __restrict__ k_codes, const uint8_t* __restrict__ v_codes,
    const float* __restrict__ k_scales, const float* __restrict__ v_scales, uint32_t code_row_stride,
    uint32_t scale_row_stride, const uint16_t* __restrict__ q, int32_t n_q_heads, int32_t n_qrows, int32_t g_shift,
    const int32_t* __restrict__ table, int64_t table_stride, const int32_t* __restrict__ seq_lens,
    int32_t max_seq_len, int32_t n_split, int32_t chunk, int32_t split_stride, float qk_scale_log2,
    int32_t key_trim, int32_t window, int32_t n_col_groups, uint32_t max_row, int32_t* __restrict__ header,
    float* __restrict__ part_o, float* __restrict__ part_lse, FoldKernelArgs fold_args) {
  constexpr int D = C::D, NT = C::NT, kWaves = C::kWaves, kBlock = C::kBlock;
  constexpr int kSteps = C::kSteps, kGroupKeys = C::kGroupKeys, kRowSlots = C::kRowSlots;
  constexpr int kNB = C::kNB, kPassCols = C::kPassCols;
  // Query heads per KV head: a template value unless several rows share the tiles.
  const int G = C::MULTI ? (1 << g_shift) : C::G;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  FP8KV_MARK(0, true);
  const int n = lane & 15;
  const int j = lane >> 4;
  // Grid (8 * Hkv, ceil(n_split / 8), batch * column groups): workgroup
  // x + 8 Hkv (y + Y z) is dispatched to XCD x & 7, so the Hkv workgroups of
  // one (request, column group, split) run on one XCD, next to each other in
  // its dispatch order: they share that XCD's L2 lines of the table and of the
  // rows' scales, and the DRAM pages of each row record.
  // When n_split is not a multiple of 8, the workgroups past the last split
  // redo the last one and store nothing (no branch at the top: it would
  // split the entry block and serialize the argument loads).
  const int split_raw = 8 * (int)blockIdx.y + (int)(blockIdx.x & 7u);
  const bool owner = split_raw < n_split;
  const int split = min(split_raw, n_split - 1);
  const int g = (int)(blockIdx.x >> 3);
  const int b = C::MULTI ? (int)blockIdx.z / n_col_groups : (int)blockIdx.z;
  const int cg = C::MULTI ? (int)blockIdx.z - b * n_col_groups : 0;
  const int n_cols = G * n_qrows;  // columns of this KV head
  const int h0 = g * G;

  // The request length as a vector load, issued first: a scalar load would
  // share its wait with the kernel-argument loads and delay the table read.
  int b_lane = b;
  asm volatile("" : "+v"(b_lane));
  const int len_lane = seq_lens[b_lane];

  __shared__ __attribute__((aligned(16))) int32_t s_rows[kWaves][kRowSlots * kWave];
  __shared__ __attribute__((aligned(16))) float2 s_sc[kWaves][kRowSlots * kWave];
  __shared__ __attribute__((aligned(16))) float sm_o[kWaves][kPassCols][128];
  __shared__ float sm_m[kWaves][16];
  __shared__ float sm_l[kWaves][16];
  // The new token of an appending call, one row per request (head dim 128,
  // one workgroup round): wave 3 of split 0's workgroup of each (request, KV
  // head) quantizes its K and V rows into the pool, scores them against the
  // group's G query heads and folds the token into the split's partial as one
  // more key; the merge is then the plain one.  Waves 0-3 get their rows
  // first and would otherwise wait on the later waves' rows, and wave 3 has
  // a single key group even when a split's keys outnumber one round of the
  // waves (waves 0 and 1 take the extra groups): 15.2 against 15.5 us per
  // layer on the 48-layer 40K step with wave 0.
  constexpr bool kFold = FOLD;
  static_assert(!FOLD || (D == 128 && !C::MULTI && !C::STREAM), "the new token is folded at head dim 128, one row, one round");
  constexpr int kFE = D / kWave;  // new-token values per lane
  constexpr int kFoldWave = kWaves / 2 - 1;
  __shared__ float s_fold_lse[kFold ? C::G : 1];
  __shared__ __attribute__((aligned(16))) float s_fold_v[kFold ? D : 4];
  const bool fold = kFold && fold_args.k_new != nullptr && split_raw == 0;

  const int32_t* trow = table + (int64_t)b * table_stride;
  int key_begin = split * chunk;
  int key_bound = min(key_begin + chunk, max_seq_len);  // host-side bound on this split's keys
  int k_first = key_begin + wave * kGroupKeys;  // the wave's first key
  int rows_in[kRowSlots];
  if constexpr (!C::WINDOW) {
    // Row indices of the first group, read up to the host-side bound before
    // the length is known.  Every table entry below max_seq_len names a row
    // (clamped to the pool), so reading past the request's length is
    // harmless.  They go to LDS before the length is used, which keeps the
    // compiler from sinking the read below the length's wait.
#pragma unroll
    for (int c = 0; c < kRowSlots; ++c)
      rows_in[c] = (int)min((uint32_t)trow[max(min(k_first + c * kWave + lane, key_bound - 1), 0)], max_row);
#pragma unroll
    for (int c = 0; c < kRowSlots; ++c) s_rows[wave][c * kWave + lane] = rows_in[c];
    FP8KV_MARK(1, true);
  }

  // Q^T operand of tile t: column n is c = (cg * NT + t) * 16 + n (query row
  // c / G, head h0 + c % G); for MFMA kk the lane's eight k-slots are
  // d = 64*(kk/2) + 16*j + 8*(kk%2) + [0, 8).  Columns past the last repeat it:
  // MFMA outputs never mix columns, so they only produce values that are never
  // stored, and the loads need no branch (which would make the waits on the
  // loads issued before them inexact).
  bf16x8 qb[NT][C::kQK];
  int col_row[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int c = min((cg * NT + t) * 16 + n, n_cols - 1);
    const int i = C::MULTI ? (c >> g_shift) : 0;
    col_row[t] = i;
    const uint16_t* qrow = q + (((int64_t)b * n_qrows + i) * n_q_heads + h0 + (c - i * G)) * D + 16 * j;
#pragma unroll
    for (int kk = 0; kk < C::kQK; ++kk)
      qb[t][kk] = u4_as_bf16x8(*reinterpret_cast<const uint4*>(qrow + 64 * (kk >> 1) + 8 * (kk & 1)));
  }
  // The new token's rows and the group's query heads, in the layout of the
  // quantize-on-write kernel (E values per lane), requested now so that they
  // land with this wave's first rows.
  typedef typename LaneVec<kFE>::U fvecu;
  fvecu fk2 = {}, fv2 = {};
  fvecu fq2[kFold ? C::G : 1] = {};
  int64_t fslot = 0;
  if constexpr (kFold) {
    if (fold && wave == kFoldWave) {
      fslot = min((uint32_t)fold_args.new_slots[b], max_row);  // out-of-range slots are clamped, never followed
      const int64_t src = (int64_t)b * fold_args.new_token_stride + g * D + kFE * lane;
      fk2 = *reinterpret_cast<const fvecu*>(fold_args.k_new + src);
      fv2 = *reinterpret_cast<const fvecu*>(fold_args.v_new + src);
#pragma unroll
      for (int hh = 0; hh < C::G; ++hh)
        fq2[hh] = *reinterpret_cast<const fvecu*>(q + ((int64_t)b * n_q_heads + h0 + hh) * D + kFE * lane);
    }
  }

  // Positions: request length len; query row i sits at p_i = len - n_qrows + i
  // and sees positions [lo_i, p_i] (lo_i = p_i + 1 - window with a window).
  // With key_trim = k the last k positions (the new tokens of an appending
  // call) are left to the merge.
  const int len = min(__builtin_amdgcn_readfirstlane(len_lane), max_seq_len);
  const int first_end = min(len - n_qrows + 1, len - key_trim);  // end of the first row's keys
  int last_lo = 0;                                     // largest lowest visible position
  if constexpr (C::WINDOW) {
    const int first_lo = max(0, len - n_qrows + 1 - window);
    last_lo = max(0, len - window);
    key_begin = first_lo + split * chunk;
    key_bound = min(key_begin + chunk, len);
    k_first = key_begin + wave * kGroupKeys;
  }
  const int key_end = min(key_begin + chunk, len - key_trim);  // keys this split covers
  if constexpr (C::STREAM) {
    // A split past its request's length (the grid is sized by the longest
    // request) stores its empty partial -- o = 0, lse = -inf, which the merge
    // weights by zero -- and leaves without the wave merge.
    if (key_end <= key_begin) {
      if (owner) {
        for (int idx = threadIdx.x; idx < G * (D / 4); idx += kBlock) {
          const int col = idx / (D / 4);
          const int d = 4 * (idx - col * (D / 4));
          const int64_t ph = ((int64_t)b * n_q_heads + h0 + col) * split_stride + split;
          *reinterpret_cast<float4*>(part_o + ph * D + d) = make_float4(0.f, 0.f, 0.f, 0.f);
          if (d == 0) part_lse[ph] = -INFINITY;
        }
      }
      if (split == 0 && g == 0 && b == 0 && threadIdx.x == 0) header[0] = n_split;
      return;
    }
  }
  int cend[NT], clo[NT];  // the lane's columns see keys [clo, cend) of this split
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int p = len - n_qrows + col_row[t];
    cend[t] = min(p + 1, key_end);
    clo[t] = C::WINDOW ? max(0, p + 1 - window) : 0;
  }

  // Code addresses: row * stride (32 x 32 -> 64-bit) + the lane's bytes.  The
  // offsets stay on the global pointers so the loads are global, not flat.
  // K: key n of a 16-key block, 16-byte chunks j + 4c.  V: D/16 bytes at d = (D/16) n.
  const uint8_t* kbase = k_codes + g * D + 16 * j;
  const uint8_t* vbase = v_codes + g * D + (D / 16) * n;

  // Softmax reference of column n in log2 units (see run_groups), the sum of
  // p, and O[column 4j+i][d = kNB*n + nb].
  float m_run[NT], l_part[NT];
  f32x4 o[NT][kNB];
  auto reset = [&]() {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      m_run[t] = kNoMax;
      l_part[t] = 0.0f;
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) o[t][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  reset();

  // The wave's groups of keys.  LAZY = false: p = 2^(s - ref) against a fixed
  // reference per column, the maximum over its visible keys of the first of
  // the wave's steps in which it sees any, never rescaled -- no rescale
  // branch, and no maximum once every column has its reference.
  // LAZY = true: a running maximum, moved (with O and l rescaled) only when a
  // step's maximum passes it by more than kLazyMaxSlack.  reread: the first
  // group's row indices are read again (a second pass).
  auto run_groups = [&](auto lazyc, bool reread) {
    constexpr bool LAZY = decltype(lazyc)::value;
    int k0 = k_first;
    for (bool first = true; k0 < key_end; k0 += kWaves * kGroupKeys, first = false) {
      // 1. Row indices of the group's keys through LDS (per-wave region).
      if (C::WINDOW || !first || reread) {
#pragma unroll
        for (int c = 0; c < kRowSlots; ++c) {
          rows_in[c] = (int)min((uint32_t)trow[max(min(k0 + c * kWave + lane, key_bound - 1), 0)], max_row);
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

      // 3. Every code load of the group, in step order; non-temporal (NTL)
      //    when the pool's KV heads never share a line.
      u32x4 kr[kSteps][2][C::kKC];
      uint32_t vr[kSteps][8][C::kVW];
      {
#pragma unroll
        for (int t = 0; t < kSteps; ++t) {
          const int32_t* rw = &s_rows[wave][t * kDecodeTileKeys];
          if constexpr (C::STREAM) {
            // Whole 128-byte lines per load (measured faster for grids of
            // several rounds): K load h of 16-key block kb reads keys
            // 16 kb + 8h + (n & 7), 16-byte chunk j + 4 (n >> 3) -- 8 keys x 128 B;
            // V load q reads keys 2q + (n >> 3) (k-slot order), 16 bytes at
            // 16 (n & 7) -- 8 keys x 128 B.  Lanes n and n ^ 8 then trade the
            // halves each needs (see the swaps after the loads land).
            const int hi = n >> 3;
            const int4 va = *reinterpret_cast<const int4*>(rw + 4 * j);
            const int4 vb = *reinterpret_cast<const int4*>(rw + 16 + 4 * j);
            const int vrow[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
              for (int h = 0; h < 2; ++h) {
                const uint64_t r = (uint64_t)(uint32_t)rw[16 * kb + 8 * h + (n & 7)] * code_row_stride;
                kr[t][kb][h] = load_code16<NTL>(k_codes + g * D + r + 16 * j + 64 * hi);
              }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int row = hi ? vrow[2 * q + 1] : vrow[2 * q];
              const u32x4 u = load_code16<NTL>(v_codes + g * D + (uint64_t)(uint32_t)row * code_row_stride + 16 * (n & 7));
              vr[t][2 * q][0] = u.x;
              vr[t][2 * q][1] = u.y;
              vr[t][2 * q + 1][0] = u.z;
              vr[t][2 * q + 1][1] = u.w;
            }
          } else {
            const uint64_t r0 = (uint64_t)(uint32_t)rw[n] * code_row_stride;
            const uint64_t r1 = (uint64_t)(uint32_t)rw[16 + n] * code_row_stride;
#pragma unroll
            for (int c = 0; c < C::kKC; ++c) {
              kr[t][0][c] = load_code16<NTL>(kbase + r0 + 64 * c);
              kr[t][1][c] = load_code16<NTL>(kbase + r1 + 64 * c);
            }
            const int4 va = *reinterpret_cast<const int4*>(rw + 4 * j);
            const int4 vb = *reinterpret_cast<const int4*>(rw + 16 + 4 * j);
            const int vrow[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
#pragma unroll
            for (int r = 0; r < 8; ++r)
              load_v_words<C::kVW, NTL>(vbase + (uint64_t)(uint32_t)vrow[r] * code_row_stride, vr[t][r]);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // (With the fixed reference the K scale carries the softmax scale.)
#pragma unroll
      for (int c = 0; c < kRowSlots; ++c) s_sc[wave][c * kWave + lane] = make_float2(LAZY ? ksc[c] : ksc[c] * qk_scale_log2, vsc[c]);
      __builtin_amdgcn_wave_barrier();
      FP8KV_MARK(2, first);
      // Wave-uniform: only groups that reach past the first row's end, or start
      // below the last row's window start, need per-column masks.
      const bool masked = (k0 + kGroupKeys > min(first_end, key_end)) || (C::WINDOW && k0 < last_lo);

      // One 32-key step; st is a compile-time constant so kr/vr stay in
      // registers.  Steps are not skipped (no branch the loads could sink
      // into); keys a column does not see are masked out of its softmax.
      auto step = [&](auto stc) {
        constexpr int st = decltype(stc)::value;
        const int t0 = k0 + st * kDecodeTileKeys;
        if constexpr (C::STREAM) {
          // Whole-line loads: lane n < 8 holds its own K chunk j (load 0) and
          // chunk j of key n + 8 (load 1); lane n + 8 holds chunk j + 4 of key
          // n (load 0) and its own chunk j + 4 (load 1).  After the trade every
          // lane holds chunks j and j + 4 of key n, as the MFMA rows need.
          // V: lane n < 8 loaded bytes 16 (n & 7) .. + 15 of key 2q, lane n + 8
          // those of key 2q + 1; lane n keeps columns d = 16 (n & 7) + 8 (n >> 3)
          // .. + 7 of both keys.
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            const u32x4 l0 = kr[st][kb][0], l1 = kr[st][kb][1];
            u32x4 a, c;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              a[w] = swap8_into<0xC>(l0[w], l1[w]);
              c[w] = swap8_into<0x3>(l1[w], l0[w]);
            }
            kr[st][kb][0] = a;
            kr[st][kb][1] = c;
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t lo0 = vr[st][2 * q][0], lo1 = vr[st][2 * q][1];
            const uint32_t hi0 = vr[st][2 * q + 1][0], hi1 = vr[st][2 * q + 1][1];
            vr[st][2 * q][0] = swap8_into<0xC>(lo0, hi0);
            vr[st][2 * q][1] = swap8_into<0xC>(lo1, hi1);
            vr[st][2 * q + 1][0] = swap8_into<0x3>(hi0, lo0);
            vr[st][2 * q + 1][1] = swap8_into<0x3>(hi1, lo1);
          }
        }
        // S^T = K * Q^T: lane (n, j) holds chunks j + 4c of keys n (block 0)
        // and 16+n (block 1).  Each K operand is widened once for all tiles.
        f32x4 s0[NT], s1[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) s0[t] = s1[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < C::kQK; ++kk) {
          const u32x4 w0 = kr[st][0][kk >> 1], w1 = kr[st][1][kk >> 1];
          const bf16x8 a0 = (kk & 1) ? C::Code::widen8(w0.z, w0.w) : C::Code::widen8(w0.x, w0.y);
          const bf16x8 a1 = (kk & 1) ? C::Code::widen8(w1.z, w1.w) : C::Code::widen8(w1.x, w1.y);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            s0[t] = mfma16x16x32(a0, qb[t][kk], s0[t]);
            s1[t] = mfma16x16x32(a1, qb[t][kk], s1[t]);
          }
        }
        const float2* scp = &s_sc[wave][st * kDecodeTileKeys];
        const float4 c01 = *reinterpret_cast<const float4*>(&scp[4 * j]);
        const float4 c23 = *reinterpret_cast<const float4*>(&scp[4 * j + 2]);
        const float4 c45 = *reinterpret_cast<const float4*>(&scp[16 + 4 * j]);
        const float4 c67 = *reinterpret_cast<const float4*>(&scp[16 + 4 * j + 2]);

        bf16x8 pa[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          // Scores in log2 units for column n, keys step_key(j, r); keys the
          // column does not see get -inf.
          const float raw[8] = {s0[t][0], s0[t][1], s0[t][2], s0[t][3], s1[t][0], s1[t][1], s1[t][2], s1[t][3]};
          const float kq[8] = {c01.x, c01.z, c23.x, c23.z, c45.x, c45.z, c67.x, c67.z};
          auto mask = [&](float (&x)[8]) {
            if (masked) {
#pragma unroll
              for (int r = 0; r < 8; ++r) {
                const int key = t0 + step_key(j, r);
                const bool vis = key < cend[t] && (!C::WINDOW || key >= clo[t]);
                x[r] = vis ? x[r] : -INFINITY;
              }
            }
          };
          auto column_max = [&](const float (&x)[8]) {
            const float m = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
            return max_over_row_groups(m);
          };
          float p[8];
          if constexpr (LAZY) {
            float sv[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) sv[r] = raw[r] * kq[r] * qk_scale_log2;
            mask(sv);
            const float tmax = column_max(sv);
            // Lazy maximum: move it (and rescale O and l) only when this step's
            // maximum exceeds it by more than the slack; otherwise p <= 2^slack.
            // A column with no visible key keeps m_run = kNoMax and gets p = 0.
            if (__any(tmax > m_run[t] + kLazyMaxSlack)) {
              const float m_new = fmaxf(m_run[t], tmax);
              const float alpha = fast_exp2(m_run[t] - m_new);
              m_run[t] = m_new;
              l_part[t] *= alpha;
              float ai[4];
#pragma unroll
              for (int i = 0; i < 4; ++i) ai[i] = __shfl(alpha, 4 * j + i);
#pragma unroll
              for (int nb = 0; nb < kNB; ++nb) {
#pragma unroll
                for (int i = 0; i < 4; ++i) o[t][nb][i] *= ai[i];
              }
            }
#pragma unroll
            for (int r = 0; r < 8; ++r) p[r] = fast_exp2(sv[r] - m_run[t]);
          } else {
            if (__any(m_run[t] == kNoMax)) {
              // A column without a reference takes this step's maximum over
              // its visible keys (it keeps kNoMax if it sees none); its O and l
              // are still zero.
              float sv[8];
#pragma unroll
              for (int r = 0; r < 8; ++r) sv[r] = raw[r] * kq[r];
              mask(sv);
              const float tmax = column_max(sv);
              m_run[t] = (m_run[t] == kNoMax) ? fmaxf(tmax, kNoMax) : m_run[t];
            }
            float x[8];  // score - reference
#pragma unroll
            for (int r = 0; r < 8; ++r) x[r] = fmaf(raw[r], kq[r], -m_run[t]);
            mask(x);
#pragma unroll
            for (int r = 0; r < 8; ++r) p[r] = fast_exp2(x[r]);
          }
          l_part[t] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
          // P' = p * v_scale as the bf16 A operand (row = column n, k-slots = keys).
          const uint4 pu = make_uint4(f32x2_to_bf16x2(p[0] * c01.y, p[1] * c01.w), f32x2_to_bf16x2(p[2] * c23.y, p[3] * c23.w),
                                      f32x2_to_bf16x2(p[4] * c45.y, p[5] * c45.w), f32x2_to_bf16x2(p[6] * c67.y, p[7] * c67.w));
          pa[t] = u4_as_bf16x8(pu);
        }

        // 4. V operand for column block nb: byte nb of each key's D/16 bytes,
        //    i.e. V[key][d = kNB*n + nb] for the lane's 8 keys, shared by all
        //    tiles.
#pragma unroll
        for (int w = 0; w < C::kVW; ++w) {
          // pr[q][h]: keys 2q and 2q+1 at channels 4w + 2h and 4w + 2h + 1,
          // interleaved -- one byte permute per dword, and the widening
          // convert picks the channel's half.
          uint32_t pr[4][2];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            pr[q][0] = __builtin_amdgcn_perm(vr[st][2 * q + 1][w], vr[st][2 * q][w], 0x05010400u);
            pr[q][1] = __builtin_amdgcn_perm(vr[st][2 * q + 1][w], vr[st][2 * q][w], 0x07030602u);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int h = e >> 1;
            const bf16x8 vb = (e & 1) ? C::Code::template widen_pairs<true>(pr[0][h], pr[1][h], pr[2][h], pr[3][h])
                                      : C::Code::template widen_pairs<false>(pr[0][h], pr[1][h], pr[2][h], pr[3][h]);
#pragma unroll
            for (int t = 0; t < NT; ++t) o[t][4 * w + e] = mfma16x16x32(pa[t], vb, o[t][4 * w + e]);
          }
        }
      };
      step(std::integral_constant<int, 0>{});
      FP8KV_MARK(3, first);
      if constexpr (kSteps > 1) step(std::integral_constant<int, 1>{});
      if constexpr (kSteps > 2) step(std::integral_constant<int, 2>{});
      if constexpr (kSteps > 3) step(std::integral_constant<int, 3>{});
      __builtin_amdgcn_wave_barrier();  // this group's LDS is consumed before the next overwrites it
    }
  };
  if constexpr (D == 256) {
    // The registers are full at D = 256: a second pass's code would spill.
    run_groups(std::true_type{}, false);
  } else {
    run_groups(std::false_type{}, false);
    // A key far enough above the reference overflows p, l or O and leaves a
    // non-finite value (inf and NaN absorb); finite l and O mean the result
    // is a running maximum's, up to rounding.  Otherwise the wave's keys are
    // read and summed again with the running maximum.
    // One sum over l and O is finite exactly when they all are, or else
    // overflows itself, which only sends the wave round again.
    float total = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      total += l_part[t];
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) total += o[t][nb][i];
    }
    // The test is on the bits, out of the compiler's sight: as a floating-
    // point class test it could be folded away for NaN (the build assumes no
    // NaN operands), and inf * 0 in the MFMAs makes NaN from an overflow.
    uint32_t total_bits = __float_as_uint(total);
    asm volatile("" : "+v"(total_bits));
    if (__any((total_bits & 0x7fffffffu) >= 0x7f800000u)) {
      reset();
      run_groups(std::true_type{}, true);
    }
  }
  FP8KV_MARK(4, true);

  if constexpr (kFold) {
    if (fold && wave == kFoldWave) {
      // Quantize the new token's rows into its pool row; its score against
      // each query head (log2 units) and its value, from the decoded codes,
      // go to LDS for the partial below.
      const NewTokenCodes<kFE> nt = quantize_new_token<kFE, C::F>(fk2, fv2);
#pragma unroll
      for (int hh = 0; hh < C::G; ++hh) {
        float qx[kFE];
#pragma unroll
        for (int e = 0; e < kFE; e += 2) {
          qx[e] = bf16lo_to_f32(fq2[hh][e / 2]);
          qx[e + 1] = bf16hi_to_f32(fq2[hh][e / 2]);
        }
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < kFE; ++e) part += qx[e] * nt.kd[e];
        const float dot = wave_sum(part);
        if (lane == 0) s_fold_lse[hh] = dot * nt.sk * qk_scale_log2;
      }
#pragma unroll
      for (int e = 0; e < kFE; ++e) s_fold_v[kFE * lane + e] = nt.vd[e] * nt.sv;
      uint8_t* kdst = const_cast<uint8_t*>(k_codes) + fslot * code_row_stride + g * D + kFE * lane;
      uint8_t* vdst = const_cast<uint8_t*>(v_codes) + fslot * code_row_stride + g * D + kFE * lane;
      static_assert(kFE == 2, "two codes per lane at head dim 128");
      *reinterpret_cast<uint16_t*>(kdst) = (uint16_t)nt.kc;
      *reinterpret_cast<uint16_t*>(vdst) = (uint16_t)nt.vc;
      if (lane == 0) {
        const_cast<float*>(k_scales)[fslot * scale_row_stride + g] = nt.sk;
        const_cast<float*>(v_scales)[fslot * scale_row_stride + g] = nt.sv;
      }
    }
  }

  // Merge the waves of this workgroup into one partial per column, one pass
  // per (tile, 128 of the D columns of O).  In pass half, LDS column
  // d' = 8 n' + e holds d = kNB n' + 8 half + e.
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float l_tot = sum_over_row_groups(l_part[t]);
#pragma unroll
    for (int half = 0; half < D / 128; ++half) {
      if (t + half > 0) __syncthreads();  // the previous pass has read LDS
      if (j == 0 && n < kPassCols) {
        sm_m[wave][n] = m_run[t];
        sm_l[wave][n] = l_tot;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int col = 4 * j + i;
        if (col < kPassCols) {
          float* dst = &sm_o[wave][col][8 * n];
          const int e0 = 8 * half;
          *reinterpret_cast<float4*>(dst) = make_float4(o[t][e0][i], o[t][e0 + 1][i], o[t][e0 + 2][i], o[t][e0 + 3][i]);
          *reinterpret_cast<float4*>(dst + 4) =
              make_float4(o[t][e0 + 4][i], o[t][e0 + 5][i], o[t][e0 + 6][i], o[t][e0 + 7][i]);
        }
      }
      __syncthreads();
      for (int idx = threadIdx.x; idx < kPassCols * 32; idx += kBlock) {
        const int col = idx >> 5;
        const int c = (cg * NT + t) * 16 + col;
        if (c >= n_cols || !owner) continue;
        const int i = C::MULTI ? (c >> g_shift) : 0;
        const int dp = 4 * (idx & 31);
        // LDS column 8 n' + e holds lane n''s O column: d = kNB n' + 8 half + e,
        // or 16 (n' & 7) + 8 (n' >> 3) + e for the whole-line V loads.
        const int d = C::STREAM ? 16 * ((dp >> 3) & 7) + 8 * (dp >> 6) + (dp & 7)
                                : kNB * (dp >> 3) + 8 * half + (dp & 7);
        float M = sm_m[0][col];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm_m[w][col]);
        if constexpr (kFold) {
          if (fold) M = fmaxf(M, s_fold_lse[col]);
        }
        float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
        float den = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const float wt = fast_exp2(sm_m[w][col] - M);
          const float4 v = *reinterpret_cast<const float4*>(&sm_o[w][col][dp]);
          num.x += wt * v.x;
          num.y += wt * v.y;
          num.z += wt * v.z;
          num.w += wt * v.w;
          den += wt * sm_l[w][col];
        }
        if constexpr (kFold) {
          if (fold) {  // the new token: one key of weight 2^(score - M) and value v
            const float wt = fast_exp2(s_fold_lse[col] - M);
            const float4 v = *reinterpret_cast<const float4*>(&s_fold_v[d]);
            num.x += wt * v.x;
            num.y += wt * v.y;
            num.z += wt * v.z;
            num.w += wt * v.w;
            den += wt;
          }
        }
        const float inv = (den > 0.f) ? 1.0f / den : 0.0f;
        const int64_t bh = ((int64_t)b * n_qrows + i) * n_q_heads + h0 + (c - i * G);
        const int64_t ph = bh * split_stride + split;
        *reinterpret_cast<float4*>(part_o + ph * D + d) = make_float4(num.x * inv, num.y * inv, num.z * inv, num.w * inv);
        if (half == 0 && dp == 0) part_lse[ph] = (den > 0.f) ? M + log2f(den) : -INFINITY;
      }
    }
  }
  // The split count for a merge launched without one.  Written last: a branch
  // at the top would split the entry block and serialize the argument loads
  // ahead of the first table read.
  FP8KV_MARK(5, true);
  if (split == 0 && g == 0 && cg == 0 && b == 0 && threadIdx.x == 0) header[0] = n_split;
}

// Stage 2: out[b][h] = sum_s 2^(lse_s - M) o_s / sum_s 2^(lse_s - M) over the
// splits of (b, h).  One workgroup per (request, query row, query head) of
// W waves (8; 2, 4 and 16 were measured slower on the 32K step); wave w takes
// splits w, w+W, ...: it loads their lse and o vectors together (clamped
// indices, no branches), keeps its own maximum, and the waves combine through
// LDS -- a single memory round trip.  Lane l owns d = E*l .. E*l + E-1
// (E = D / 64).
//
// With APPEND (the appending calls whose new tokens stage 1 does not take:
// several query rows, head dim 256, or several workgroup rounds), the
// request's last n_qrows positions are new tokens, left out of stage 1; in
// the workgroup of query row i, wave j <= i takes new token j:
// it quantizes the token's bf16 K and V rows of the head group exactly as the
// quantize-on-write kernel does (same codec functions), scores q against the
// decoded codes, and, when the token lies inside the row's window, folds it in
// as a single-key partial (o = s_v * decode(v), lse = the score).  The
// workgroup of the group's first query head and the last query row writes the
// codes and scales to the tokens' rows new_slots[b][j]; every load of the
// kernel is independent (one round trip).
#ifndef FP8KV_MERGE_WAVES
#define FP8KV_MERGE_WAVES 8
#endif
constexpr int kMergeWaves = FP8KV_MERGE_WAVES;
constexpr int kMergeBlock = kMergeWaves * kWave;
constexpr int kMergeBatch = 64 / kMergeWaves;  // splits per wave loaded at once (64 per workgroup)
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
  int32_t n_qrows;  // new tokens (and query rows) per request
  int32_t window;   // 0: every new token j <= i is visible to query row i
};

template <int D, bool APPEND, int F = kE4M3>
__global__ __launch_bounds__(kMergeBlock) void decode_merge_kernel(const int32_t* __restrict__ header,
                                                                  const float* __restrict__ part_o,
                                                                  const float* __restrict__ part_lse,
                                                                  int32_t split_stride, int32_t n_split_arg,
                                                                  int32_t n_q_heads, AppendKernelArgs app,
                                                                  uint16_t* __restrict__ out) {
  constexpr int E = D / kWave;
  typedef typename LaneVec<E>::F vecf;
  typedef typename LaneVec<E>::U vecu;
  __shared__ float s_m[kMergeWaves];
  __shared__ float s_den[kMergeWaves];
  __shared__ vecf s_acc[kMergeWaves][kWave];
  const int64_t bh = blockIdx.x;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  // A split count read from the workspace is clamped to its capacity, so a
  // workspace that no stage 1 wrote cannot send the loads past it; a count of
  // 0 loads split 0 (inside the workspace), folds nothing and stores zeros.
  const int n_split = n_split_arg >= 0 ? n_split_arg : min(max(header[0], 0), split_stride);
  const int last_split = max(n_split - 1, 0);
  const float* lse_p = part_lse + bh * split_stride;
  const float* po = part_o + bh * split_stride * D + E * lane;

  // The new token's inputs: its bf16 K/V values at d = E*lane + [0, E), and q.
  vecu k2 = {}, v2 = {}, q2 = {};
  int64_t slot = 0;
  int64_t b = 0, g = 0;
  // Query row i of request b; wave j < n_new takes new token j (position
  // seq_lens[b] - n_qrows + j), visible to row i when j <= i and inside the
  // window.
  int qi = 0, n_new = 0;
  bool visible = false;
  if constexpr (APPEND) {
    const int64_t bq = bh / n_q_heads;
    b = bq / app.n_qrows;
    qi = (int)(bq - b * app.n_qrows);
    n_new = qi + 1;
    const int h = (int)(bh % n_q_heads);
    g = h / (n_q_heads / app.n_kv_heads);
    visible = wave < n_new && (app.window == 0 || qi - wave < app.window);
    if (wave < n_new) {
      const int64_t tok = b * app.n_qrows + wave;
      slot = min((uint32_t)app.new_slots[tok], app.max_row);  // out-of-range slots are clamped, never followed
      k2 = *reinterpret_cast<const vecu*>(app.k_new + tok * app.new_token_stride + g * D + E * lane);
      v2 = *reinterpret_cast<const vecu*>(app.v_new + tok * app.new_token_stride + g * D + E * lane);
      q2 = *reinterpret_cast<const vecu*>(app.q + bh * D + E * lane);
    }
  }

  float m_w = -INFINITY, den = 0.f;
  vecf acc = {};
  // One batch of splits: wave w takes splits base + w + 4i, loaded together
  // (clamped indices, no branches) and folded into (m_w, den, acc).
  float lr[kMergeBatch];
  vecf v[kMergeBatch];
  auto load_batch = [&](int base) {
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      const int sidx = min(base + wave + kMergeWaves * i, last_split);
      lr[i] = lse_p[sidx];
      v[i] = *reinterpret_cast<const vecf*>(po + (int64_t)sidx * D);
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
      acc *= a;
      den *= a;
      m_w = mx;
#pragma unroll
      for (int i = 0; i < kMergeBatch; ++i) {
        const float w = __builtin_amdgcn_exp2f(lr[i] - m_w);
        acc += w * v[i];
        den += w;
      }
    }
  };
  load_batch(0);  // in flight while wave 0 quantizes and scores the new token

  float lse_new = -INFINITY;
  vecf o_new = {};
  if constexpr (APPEND) {
    if (wave < n_new) {
      // Quantize the K and V rows (D values over the wave, E per lane); score
      // and value from the decoded codes, as stage 1 sees every other row.
      const NewTokenCodes<E> nt = quantize_new_token<E, F>(k2, v2);
      const uint32_t kc = nt.kc, vc = nt.vc;
      const float sk = nt.sk, sv = nt.sv;
      float qx[E];
#pragma unroll
      for (int e = 0; e < E; e += 2) {
        qx[e] = bf16lo_to_f32(q2[e / 2]);
        qx[e + 1] = bf16hi_to_f32(q2[e / 2]);
      }
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) part += qx[e] * nt.kd[e];
      const float dot = wave_sum(part);
      lse_new = dot * sk * app.qk_scale_log2;
#pragma unroll
      for (int e = 0; e < E; ++e) o_new[e] = nt.vd[e] * sv;
      // One workgroup per (request, KV head) stores the rows: the one of the
      // group's first query head and the last query row, which holds every
      // new token.
      if ((bh % n_q_heads) % (n_q_heads / app.n_kv_heads) == 0 && qi == app.n_qrows - 1) {
        uint8_t* kdst = app.k_codes + slot * app.code_row_stride + g * D + E * lane;
        uint8_t* vdst = app.v_codes + slot * app.code_row_stride + g * D + E * lane;
        if constexpr (E == 2) {
          *reinterpret_cast<uint16_t*>(kdst) = (uint16_t)kc;
          *reinterpret_cast<uint16_t*>(vdst) = (uint16_t)vc;
        } else {
          *reinterpret_cast<uint32_t*>(kdst) = kc;
          *reinterpret_cast<uint32_t*>(vdst) = vc;
        }
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
    if (visible) {  // the wave's new token as one more single-key partial
      const float mx = fmaxf(m_w, lse_new);
      const float a = __builtin_amdgcn_exp2f(m_w - mx);
      const float w = __builtin_amdgcn_exp2f(lse_new - mx);
      acc = acc * a + w * o_new;
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
    vecf t = {};
    float d = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kMergeWaves; ++w) {
        const float a = __builtin_amdgcn_exp2f(s_m[w] - M);
        t += a * s_acc[w][lane];
        d += a * s_den[w];
      }
    }
    const float inv = (d > 0.f) ? 1.0f / d : 0.0f;
    vecu r;
#pragma unroll
    for (int e = 0; e < E; e += 2) r[e / 2] = f32x2_to_bf16x2(t[e] * inv, t[e + 1] * inv);
    *reinterpret_cast<vecu*>(out + bh * D + E * lane) = r;
  }
}

template <class C>
hipError_t launch_stage1_cfg(const PoolView& pool, const uint16_t* q, const DecodeShape& sh, float qk_scale_log2,
                             const DecodeGeometry& geo, const DecodeWorkspace& ws, int32_t key_trim,
                             const FoldKernelArgs& fold, hipStream_t stream) {
  const int64_t z = (int64_t)sh.batch * geo.n_col_groups;
  if (z > FP8KV_MAX_DECODE_GROUPS_INTERNAL) return hipErrorInvalidValue;  // the entry points reject it first
  const dim3 grid((unsigned)(8 * pool.n_kv_heads), (unsigned)((geo.n_split + 7) / 8), (unsigned)z);
  int g_shift = 0;
  while ((1 << g_shift) < sh.n_q_heads / pool.n_kv_heads) ++g_shift;
  auto kernel = pool.line_rows ? decode_stage1_kernel<C, true, false> : decode_stage1_kernel<C, false, false>;
  if constexpr (C::D == 128 && !C::MULTI && !C::STREAM) {
    if (fold.k_new) kernel = pool.line_rows ? decode_stage1_kernel<C, true, true> : decode_stage1_kernel<C, false, true>;
  }
  hipLaunchKernelGGL(kernel, grid, dim3(C::kBlock), 0, stream, pool.k_codes, pool.v_codes,
                     pool.k_scales, pool.v_scales, (uint32_t)pool.code_row_stride, (uint32_t)pool.scale_row_stride,
                     q, sh.n_q_heads, sh.n_qrows, g_shift, sh.row_table, sh.table_stride, sh.seq_lens, sh.max_seq_len,
                     geo.n_split, geo.chunk, ws.split_stride, qk_scale_log2, key_trim, sh.window, geo.n_col_groups,
                     (uint32_t)(pool.num_rows - 1), ws.header, ws.part_o, ws.part_lse, fold);
  return hipGetLastError();
}

// One row per request: G is a template value.
template <int D, bool WINDOW, int F>
hipError_t launch_stage1_single(const PoolView& pool, const uint16_t* q, const DecodeShape& sh, float qk,
                                const DecodeGeometry& geo, const DecodeWorkspace& ws, int32_t key_trim,
                                const FoldKernelArgs& fold, hipStream_t stream) {
  // The streaming shape exists for head dim 128 without a window.
  constexpr bool kCanStream = D == 128 && !WINDOW;
  const bool st = kCanStream && geo.stream;
  switch (sh.n_q_heads / pool.n_kv_heads) {
    case 1:
      return st ? launch_stage1_cfg<Stage1<1, D, 1, false, false, F, kCanStream>>(pool, q, sh, qk, geo, ws, key_trim, fold, stream)
                : launch_stage1_cfg<Stage1<1, D, 1, false, WINDOW, F>>(pool, q, sh, qk, geo, ws, key_trim, fold, stream);
    case 2:
      return st ? launch_stage1_cfg<Stage1<2, D, 1, false, false, F, kCanStream>>(pool, q, sh, qk, geo, ws, key_trim, fold, stream)
                : launch_stage1_cfg<Stage1<2, D, 1, false, WINDOW, F>>(pool, q, sh, qk, geo, ws, key_trim, fold, stream);
    case 4:
      return st ? launch_stage1_cfg<Stage1<4, D, 1, false, false, F, kCanStream>>(pool, q, sh, qk, geo, ws, key_trim, fold, stream)
                : launch_stage1_cfg<Stage1<4, D, 1, false, WINDOW, F>>(pool, q, sh, qk, geo, ws, key_trim, fold, stream);
    case 8:
      return st ? launch_stage1_cfg<Stage1<8, D, 1, false, false, F, kCanStream>>(pool, q, sh, qk, geo, ws, key_trim, fold, stream)
                : launch_stage1_cfg<Stage1<8, D, 1, false, WINDOW, F>>(pool, q, sh, qk, geo, ws, key_trim, fold, stream);
    case 16:
      return st ? launch_stage1_cfg<Stage1<16, D, 1, false, false, F, kCanStream>>(pool, q, sh, qk, geo, ws, key_trim, fold, stream)
                : launch_stage1_cfg<Stage1<16, D, 1, false, WINDOW, F>>(pool, q, sh, qk, geo, ws, key_trim, fold, stream);
    default: return hipErrorInvalidValue;
  }
}

// Several rows per request: NT column tiles per workgroup, G at run time.
template <int D, bool WINDOW, int F>
hipError_t launch_stage1_multi(const PoolView& pool, const uint16_t* q, const DecodeShape& sh, float qk,
                               const DecodeGeometry& geo, const DecodeWorkspace& ws, int32_t key_trim,
                               const FoldKernelArgs& fold, hipStream_t stream) {
  switch (geo.col_tiles) {
    case 1: return launch_stage1_cfg<Stage1<16, D, 1, true, WINDOW, F>>(pool, q, sh, qk, geo, ws, key_trim, fold, stream);
    case 2: return launch_stage1_cfg<Stage1<16, D, 2, true, WINDOW, F>>(pool, q, sh, qk, geo, ws, key_trim, fold, stream);
    case 4:
      if constexpr (D == 128)
        return launch_stage1_cfg<Stage1<16, D, 4, true, WINDOW, F>>(pool, q, sh, qk, geo, ws, key_trim, fold, stream);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

// Head dim and window of one code format.
template <int F>
hipError_t launch_stage1_format(const PoolView& pool, const uint16_t* q, const DecodeShape& sh, float qk,
                                const DecodeGeometry& geo, const DecodeWorkspace& ws, int32_t key_trim,
                                const FoldKernelArgs& fold, hipStream_t stream) {
  const bool window = sh.window > 0;
  if (sh.n_qrows == 1 && geo.n_col_groups == 1 && geo.col_tiles == 1) {
    if (pool.head_dim == 128)
      return window ? launch_stage1_single<128, true, F>(pool, q, sh, qk, geo, ws, key_trim, fold, stream)
                    : launch_stage1_single<128, false, F>(pool, q, sh, qk, geo, ws, key_trim, fold, stream);
    if (pool.head_dim == 256)
      return window ? launch_stage1_single<256, true, F>(pool, q, sh, qk, geo, ws, key_trim, fold, stream)
                    : launch_stage1_single<256, false, F>(pool, q, sh, qk, geo, ws, key_trim, fold, stream);
    return hipErrorInvalidValue;
  }
  if (pool.head_dim == 128)
    return window ? launch_stage1_multi<128, true, F>(pool, q, sh, qk, geo, ws, key_trim, fold, stream)
                  : launch_stage1_multi<128, false, F>(pool, q, sh, qk, geo, ws, key_trim, fold, stream);
  if (pool.head_dim == 256)
    return window ? launch_stage1_multi<256, true, F>(pool, q, sh, qk, geo, ws, key_trim, fold, stream)
                  : launch_stage1_multi<256, false, F>(pool, q, sh, qk, geo, ws, key_trim, fold, stream);
  return hipErrorInvalidValue;
}

template <int D>
hipError_t launch_merge_d(int64_t n_rows_heads, const DecodeWorkspace& ws, int32_t n_split, int32_t n_q_heads,
                          uint16_t* out, hipStream_t stream) {
  hipLaunchKernelGGL((decode_merge_kernel<D, false>), dim3((unsigned)n_rows_heads), dim3(kMergeBlock), 0, stream,
                     ws.header, ws.part_o, ws.part_lse, ws.split_stride, n_split, n_q_heads, AppendKernelArgs{}, out);
  return hipGetLastError();
}

}  // namespace

// Column tiles per workgroup: beyond them, further column groups re-read the
// rows (mostly from L2).  At D = 128, two 8-wave workgroups of 2 tiles beat
// one 4-wave workgroup of 4 tiles (64 columns, 32K keys: 23.9 vs 26.6 us):
// the wide shape's 512 registers per wave leave one wave per SIMD.
#ifndef FP8KV_DECODE_MAX_TILES_128
#define FP8KV_DECODE_MAX_TILES_128 2
#endif
#ifndef FP8KV_DECODE_MAX_TILES_256
#define FP8KV_DECODE_MAX_TILES_256 2
#endif
int32_t decode_max_col_tiles(int32_t head_dim) {
  return head_dim == 128 ? FP8KV_DECODE_MAX_TILES_128 : FP8KV_DECODE_MAX_TILES_256;
}

bool decode_stage1_takes_new_token(const PoolView& pool, const DecodeShape& sh, const DecodeGeometry& geo) {
  // The instantiations that fold it: head dim 128, one query row per request
  // (one 16-column tile), one workgroup round (not the streaming shape).
  return pool.head_dim == 128 && sh.n_qrows == 1 && geo.n_col_groups == 1 && geo.col_tiles == 1 && !geo.stream;
}

hipError_t launch_decode_stage1(const PoolView& pool, const uint16_t* q, const DecodeShape& sh, float sm_scale,
                                const DecodeGeometry& geo, const DecodeWorkspace& ws, int32_t key_trim,
                                const AppendArgs* fold, hipStream_t stream) {
  const float qk = sm_scale * kLog2e;
  if (fold && (!decode_stage1_takes_new_token(pool, sh, geo) || key_trim != 1)) return hipErrorInvalidValue;
  const FoldKernelArgs fa = fold ? FoldKernelArgs{fold->k_new, fold->v_new, fold->new_token_stride, fold->new_slots}
                                 : FoldKernelArgs{nullptr, nullptr, 0, nullptr};
  if (pool.format == kInt8) return launch_stage1_format<kInt8>(pool, q, sh, qk, geo, ws, key_trim, fa, stream);
  if (pool.format == kE4M3) return launch_stage1_format<kE4M3>(pool, q, sh, qk, geo, ws, key_trim, fa, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_merge(int64_t n_rows_heads, int32_t head_dim, const DecodeWorkspace& ws, int32_t n_split,
                               uint16_t* out, hipStream_t stream) {
  if (head_dim == 128) return launch_merge_d<128>(n_rows_heads, ws, n_split, 1, out, stream);
  if (head_dim == 256) return launch_merge_d<256>(n_rows_heads, ws, n_split, 1, out, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_merge_append(const PoolView& pool, int32_t batch, int32_t n_q_heads, const DecodeWorkspace& ws,
                                      int32_t n_split, const AppendArgs& app, uint16_t* out, hipStream_t stream) {
  if (app.n_qrows < 1 || app.n_qrows > kMergeWaves) return hipErrorInvalidValue;  // one wave per new token
  const AppendKernelArgs a{app.q, app.k_new, app.v_new, app.new_token_stride, app.new_slots,
                           pool.k_codes, pool.v_codes, pool.k_scales, pool.v_scales,
                           pool.code_row_stride, pool.scale_row_stride, pool.n_kv_heads,
                           (uint32_t)(pool.num_rows - 1), app.sm_scale * kLog2e, app.n_qrows, app.window};
  const dim3 grid((unsigned)((int64_t)batch * app.n_qrows * n_q_heads));
  const bool i8 = pool.format == kInt8;
  if (pool.head_dim == 128 && !i8)
    hipLaunchKernelGGL((decode_merge_kernel<128, true, kE4M3>), grid, dim3(kMergeBlock), 0, stream, ws.header,
                       ws.part_o, ws.part_lse, ws.split_stride, n_split, n_q_heads, a, out);
  else if (pool.head_dim == 128 && i8)
    hipLaunchKernelGGL((decode_merge_kernel<128, true, kInt8>), grid, dim3(kMergeBlock), 0, stream, ws.header,
                       ws.part_o, ws.part_lse, ws.split_stride, n_split, n_q_heads, a, out);
  else if (pool.head_dim == 256 && !i8)
    hipLaunchKernelGGL((decode_merge_kernel<256, true, kE4M3>), grid, dim3(kMergeBlock), 0, stream, ws.header,
                       ws.part_o, ws.part_lse, ws.split_stride, n_split, n_q_heads, a, out);
  else if (pool.head_dim == 256 && i8)
    hipLaunchKernelGGL((decode_merge_kernel<256, true, kInt8>), grid, dim3(kMergeBlock), 0, stream, ws.header,
                       ws.part_o, ws.part_lse, ws.split_stride, n_split, n_q_heads, a, out);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace fp8kv

#ifdef FP8KV_WAVE_TIMELINE
// Measurement build: copy the first n stage-1 timeline slots to host memory /
// clear all of them.  0 on success, else the HIP error code.
extern "C" int fp8kv_timeline_read(unsigned long long* host, long n) {
  if (!host || n < 0 || n > (long)(fp8kv::kTimelineWorkgroups * 64)) return (int)hipErrorInvalidValue;
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(fp8kv::fp8kv_timeline), n * sizeof(unsigned long long), 0,
                                  hipMemcpyDeviceToHost);
}
extern "C" int fp8kv_timeline_clear() {
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(fp8kv::fp8kv_timeline));
  if (e != hipSuccess) return (int)e;
  return (int)hipMemset(p, 0, sizeof(unsigned long long) * fp8kv::kTimelineWorkgroups * 64);
}
#endif
