// fp8kv_device.h -- device-side helpers shared by the gfx950 kernels of libfp8kv.
//
// Everything here is CDNA4-specific: wave64, the packed FP8 <-> f32 / bf16
// converts added for OCP E4M3FN on gfx950, and the bf16 MFMA 16x16x32 layout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8kv_launch.h"

namespace fp8kv {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kHeadDim = 128;
constexpr int kWave = 64;

// bf16 bit pattern -> f32 (exact widening).
__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two E4M3FN codes (bytes 0,1 or 2,3 of w) -> two bf16 packed in one dword.
// Every finite E4M3FN value is exact in bf16, so this is an exact widening.
// The scaled convert with scale 1.0 leaves values unchanged.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
  return __builtin_bit_cast(uint32_t, r);
}

// Four E4M3FN codes in one dword -> bf16 x4 in two dwords (byte k -> element k).
__device__ __forceinline__ uint2 fp8x4_to_bf16x4(uint32_t w) {
  return make_uint2(fp8x2_to_bf16x2<false>(w), fp8x2_to_bf16x2<true>(w));
}

// Eight codes (two dwords) -> MFMA bf16x8 operand (byte k -> element k).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  uint2 a = fp8x4_to_bf16x4(lo), b = fp8x4_to_bf16x4(hi);
  uint4 u = make_uint4(a.x, a.y, b.x, b.y);
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ bf16x8 u4_as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// Two f32 -> two bf16 (round to nearest even) packed in one dword.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
  bf16x2 r = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, r);
}

// Two f32 -> two E4M3FN codes written into half HI of `old` (round to
// nearest even; callers clamp to +-448 first so saturation is explicit).
template <bool HI>
__device__ __forceinline__ uint32_t f32x2_to_fp8x2(float a, float b, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}

// Quantize-on-write of one element of a row whose absolute maximum is amax:
// s = fl32(amax / 448) (an IEEE division: the library is built with correctly
// rounded fp32 division), then fl32(x / s) clamped to the E4M3FN range; the
// hardware convert (f32x2_to_fp8x2) rounds that to nearest even.  An all-zero
// row keeps s = 0 and passes x through, so its codes are signed zeros.  Every
// writer of codes goes through these two functions.
__device__ __forceinline__ float e4m3_row_scale(float amax) { return amax / 448.0f; }
__device__ __forceinline__ float e4m3_prescaled(float x, float amax, float s) {
  const float q = (amax == 0.0f) ? x : x / s;
  return fminf(fmaxf(q, -448.0f), 448.0f);
}

// Four E4M3FN codes in one dword -> four f32.
__device__ __forceinline__ void fp8x4_to_f32x4(uint32_t w, float* o) {
  f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  o[0] = a.x; o[1] = a.y; o[2] = b.x; o[3] = b.y;
}

// Byte k of w as a signed INT8 code, exactly as f32.
__device__ __forceinline__ float i8_at(uint32_t w, int k) { return (float)(int8_t)(uint8_t)(w >> (8 * k)); }

// KV code formats (the values of fp8kv_pool_layer.code_format).
enum CodeFormat : int { kE4M3 = 0, kInt8 = 1 };

// Per-format quantize-on-write and widening.  scale(amax) is the row scale;
// prescale(x, amax, s) is the value handed to pack2 (E4M3: x/s clamped to the
// format's range, rounded to nearest even by the hardware convert; INT8: x/s
// rounded half to even and clamped to +-127); an all-zero row has s = 0 and
// zero codes.  widen8 turns eight code bytes into an exact bf16x8 MFMA
// operand (every E4M3FN value and every integer up to 127 is exact in bf16);
// widen4 gives four f32.
template <int F>
struct Codec;

template <>
struct Codec<kE4M3> {
  static __device__ __forceinline__ float scale(float amax) { return e4m3_row_scale(amax); }
  static __device__ __forceinline__ float prescale(float x, float amax, float s) { return e4m3_prescaled(x, amax, s); }
  template <bool HI>
  static __device__ __forceinline__ uint32_t pack2(float a, float b, uint32_t old) {
    return f32x2_to_fp8x2<HI>(a, b, old);
  }
  static __device__ __forceinline__ bf16x8 widen8(uint32_t lo, uint32_t hi) { return fp8x8_to_bf16x8(lo, hi); }
  // Four dwords of two keys' codes at two channels each ([a c b d]: key 0 and
  // key 1 at channel 0, then at channel 1) -> the eight keys at channel HI.
  template <bool HI>
  static __device__ __forceinline__ bf16x8 widen_pairs(uint32_t p0, uint32_t p1, uint32_t p2, uint32_t p3) {
    const uint4 u = make_uint4(fp8x2_to_bf16x2<HI>(p0), fp8x2_to_bf16x2<HI>(p1), fp8x2_to_bf16x2<HI>(p2),
                               fp8x2_to_bf16x2<HI>(p3));
    return __builtin_bit_cast(bf16x8, u);
  }
  static __device__ __forceinline__ void widen4(uint32_t w, float* o) { fp8x4_to_f32x4(w, o); }
};

template <>
struct Codec<kInt8> {
  static __device__ __forceinline__ float scale(float amax) { return amax / 127.0f; }
  static __device__ __forceinline__ float prescale(float x, float amax, float s) {
    return (amax == 0.0f) ? 0.0f : __builtin_rintf(fminf(fmaxf(x / s, -127.0f), 127.0f));
  }
  template <bool HI>
  static __device__ __forceinline__ uint32_t pack2(float a, float b, uint32_t old) {
    const uint32_t v = ((uint32_t)(int)a & 0xffu) | (((uint32_t)(int)b & 0xffu) << 8);
    return HI ? ((old & 0x0000ffffu) | (v << 16)) : ((old & 0xffff0000u) | v);
  }
  static __device__ __forceinline__ bf16x8 widen8(uint32_t lo, uint32_t hi) {
    const uint4 u = make_uint4(f32x2_to_bf16x2(i8_at(lo, 0), i8_at(lo, 1)), f32x2_to_bf16x2(i8_at(lo, 2), i8_at(lo, 3)),
                               f32x2_to_bf16x2(i8_at(hi, 0), i8_at(hi, 1)), f32x2_to_bf16x2(i8_at(hi, 2), i8_at(hi, 3)));
    return __builtin_bit_cast(bf16x8, u);
  }
  template <bool HI>
  static __device__ __forceinline__ bf16x8 widen_pairs(uint32_t p0, uint32_t p1, uint32_t p2, uint32_t p3) {
    constexpr int b = HI ? 2 : 0;
    const uint4 u = make_uint4(f32x2_to_bf16x2(i8_at(p0, b), i8_at(p0, b + 1)), f32x2_to_bf16x2(i8_at(p1, b), i8_at(p1, b + 1)),
                               f32x2_to_bf16x2(i8_at(p2, b), i8_at(p2, b + 1)), f32x2_to_bf16x2(i8_at(p3, b), i8_at(p3, b + 1)));
    return __builtin_bit_cast(bf16x8, u);
  }
  static __device__ __forceinline__ void widen4(uint32_t w, float* o) {
    o[0] = i8_at(w, 0); o[1] = i8_at(w, 1); o[2] = i8_at(w, 2); o[3] = i8_at(w, 3);
  }
};

// v_mfma_f32_16x16x32_bf16: D(16x16) += A(16x32) * B(32x16).
// Lane l supplies row (l % 16) of A and column (l % 16) of B, each as eight
// consecutive k-slots of k-group (l / 16); it receives D rows 4*(l/16)+i,
// column l % 16, i = 0..3.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Maximum over the four 16-lane rows of the wave (lanes n, n+16, n+32, n+48),
// returned to all four.  gfx950's row swaps keep this out of LDS:
// permlane16_swap(x, x) yields rows (0,0,2,2) and (1,1,3,3) of x,
// permlane32_swap(y, y) yields its low and high halves.
__device__ __forceinline__ float max_over_row_groups(float x) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(a.x), __uint_as_float(a.y));
  const u32x2 b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(b.x), __uint_as_float(b.y));
}

// Sum over the four 16-lane rows of the wave, returned to all four (same row
// swaps as max_over_row_groups).
__device__ __forceinline__ float sum_over_row_groups(float x) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a.x) + __uint_as_float(a.y);
  const u32x2 b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b.x) + __uint_as_float(b.y);
}

// Full-wave reductions without LDS: DPP within each 16-lane row (quad
// permutes, then the half-row and row mirrors, each pairing two groups that
// already hold equal values), then the row swaps across rows.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;  // lane i <-> 7-i within 8
constexpr int kDppRowMirror = 0x140;      // lane i <-> 15-i within 16

__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f32<kDppQuadXor1>(x));
  x = fmaxf(x, dpp_f32<kDppQuadXor2>(x));
  x = fmaxf(x, dpp_f32<kDppRowHalfMirror>(x));
  x = fmaxf(x, dpp_f32<kDppRowMirror>(x));
  return max_over_row_groups(x);
}
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_f32<kDppQuadXor1>(x);
  x += dpp_f32<kDppQuadXor2>(x);
  x += dpp_f32<kDppRowHalfMirror>(x);
  x += dpp_f32<kDppRowMirror>(x);
  return sum_over_row_groups(x);
}

}  // namespace fp8kv
