// Element encode / decode helpers shared by the codec kernels (quantize,
// dequantize, and their axis-0 forms).  Internal to the HIP sources.
//
// Encode follows the "Bit Layout" page (mxfp4community.com), section
// "Reference encode and decode", with the exponent floor taken exactly:
//   amax -> e = clip(floor(log2 amax) - emax, -127, 127) -> byte e + 127,
//   y = |x| * 2^-e, nearest grid magnitude with ties to the smaller one,
//   saturation at the top of the grid, sign bit iff x < 0.
// Rounding, fast path: gfx950's v_cvt_scalef32_pk_{fp4,fp8}_f32 compute the
// round-to-nearest-even code of x / s for a float scale s (checked on the
// hardware for every normal power-of-two scale), saturating for FP4 and
// overflowing to NaN for FP8 (so |x| is clamped to 448 * 2^e first).  Nearest
// with ties to the smaller magnitude differs from nearest-even only at exact
// midpoints, and a midpoint has at most 2 (E2M1) / 4 (E4M3) significant bits:
// its 21 / 19 low mantissa bits are zero.  -0.0 has them zero too.  So a
// kernel may take the fast path for a group of elements none of which has
// those bits zero (and whose block scale is not near the bottom of the
// range, where f32 subnormals and a subnormal scale appear).
// Rounding, exact path: on the bit pattern of y, adding (half step - 1) and
// truncating the mantissa is round-to-nearest with ties down in the normal
// binades of the element format; the subnormal range (uniform spacing) uses
// ceil(y / spacing - 1/2), which also rounds ties down.
//
// Decode follows the same page, sections "The E8M0 shared scale" (value
// 2^(byte-127), byte 0xFF poisons the block to NaN) and "Reference encode and
// decode" (sign x table[magnitude] x scale, exact).  E4M3 codes 0x7F / 0xFF
// are f8E4M3FN NaN.  Without tables: placing the element's exponent and
// mantissa bits at the top of a float32 mantissa field and multiplying by a
// power of two reproduces the element value exactly (E2M1: magnitude bits <<
// 22, times 2^126; E4M3: magnitude bits << 20, times 2^120), subnormal element
// codes included, because f32 arithmetic keeps denormals (IEEE mode, no
// flushing).  The second multiply by the block scale is exact as well.
#pragma once

#include "mx_internal.h"

namespace mx {
namespace codec {

constexpr uint32_t kNaN = 0x7FC00000u;

template <int ELEM>
struct Fmt;

// E2M1: magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}; normal binades start at 1.0.
template <>
struct Fmt<kE2M1> {
  static constexpr int kEmax = 2;
  static constexpr int kSignShift = 3;
  static constexpr uint32_t kNormalMin = 0x3F800000u;  // 1.0
  static constexpr int kShift = 22;                    // 23 - 1 mantissa bit
  static constexpr uint32_t kHalfMinus1 = (1u << (kShift - 1)) - 1u;
  static constexpr uint32_t kCodeOffset = 252u;        // (127 - 1) << 1: q(1.0) - code(1.0)
  static constexpr uint32_t kTopQ = 259u;              // q of 6.0
  static constexpr float kInvSpacing = 2.0f;           // subnormal spacing 0.5
  static constexpr int kTieShift = 11;                 // keeps the 21 low mantissa bits
};

// E4M3 (f8E4M3FN): normal binades start at 2^-6, top finite value 448.
template <>
struct Fmt<kE4M3> {
  static constexpr int kEmax = 8;
  static constexpr int kSignShift = 7;
  static constexpr uint32_t kNormalMin = 0x3C800000u;  // 2^-6
  static constexpr int kShift = 20;                    // 23 - 3 mantissa bits
  static constexpr uint32_t kHalfMinus1 = (1u << (kShift - 1)) - 1u;
  static constexpr uint32_t kCodeOffset = 960u;        // (127 - 7) << 3
  static constexpr uint32_t kTopQ = 1086u;             // q of 448 (code 0x7E)
  static constexpr float kInvSpacing = 512.0f;         // subnormal spacing 2^-9
  static constexpr int kTieShift = 13;                 // keeps the 19 low mantissa bits
};

// Magnitude index of y = |x| / 2^e (finite, y < 2^(emax+1)), ties to the
// smaller magnitude, saturating at the top of the grid.
template <int ELEM>
__device__ __forceinline__ uint32_t magnitude_index(float y) {
  using F = Fmt<ELEM>;
  const uint32_t yb = __float_as_uint(y);
  const uint32_t qn = min((yb + F::kHalfMinus1) >> F::kShift, F::kTopQ) - F::kCodeOffset;
  const uint32_t qs = (uint32_t)(int)__builtin_ceilf(__builtin_fmaf(y, F::kInvSpacing, -0.5f));
  return yb >= F::kNormalMin ? qn : qs;
}

template <int ELEM>
__device__ __forceinline__ uint32_t element_code(uint32_t xb, float inv_scale) {
  using F = Fmt<ELEM>;
  const float y = __uint_as_float(xb & 0x7FFFFFFFu) * inv_scale;  // exact: power-of-two scaling
  const uint32_t neg = xb > 0x80000000u ? (1u << F::kSignShift) : 0u;  // x < 0 (not -0.0)
  return magnitude_index<ELEM>(y) | neg;
}

typedef short v2s __attribute__((ext_vector_type(2)));
typedef float f4v __attribute__((ext_vector_type(4)));

// Codes of 4 elements by the hardware convert (fast path): E2M1 -> 16 bits,
// E4M3 -> 32 bits, element 0 lowest.
template <int ELEM>
__device__ __forceinline__ uint32_t convert4(float4 v, float scale, float clamp) {
  if (ELEM == kE2M1) {
    uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v.x, v.y, scale, 0);
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v.z, v.w, scale, 1);
  } else {
    // FP8 conversion overflows to NaN past 464 * scale: clamp to the grid top.
    const float x0 = __builtin_amdgcn_fmed3f(v.x, -clamp, clamp);
    const float x1 = __builtin_amdgcn_fmed3f(v.y, -clamp, clamp);
    const float x2 = __builtin_amdgcn_fmed3f(v.z, -clamp, clamp);
    const float x3 = __builtin_amdgcn_fmed3f(v.w, -clamp, clamp);
    v2s w = {0, 0};
    w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, x0, x1, scale, false);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, x2, x3, scale, true);
    return (uint32_t)(uint16_t)w[0] | ((uint32_t)(uint16_t)w[1] << 16);
  }
}

// Codes of 4 elements by exact integer rounding (exact path).
template <int ELEM>
__device__ __forceinline__ uint32_t round4(float4 v, float inv_scale) {
  const uint32_t c0 = element_code<ELEM>(__float_as_uint(v.x), inv_scale);
  const uint32_t c1 = element_code<ELEM>(__float_as_uint(v.y), inv_scale);
  const uint32_t c2 = element_code<ELEM>(__float_as_uint(v.z), inv_scale);
  const uint32_t c3 = element_code<ELEM>(__float_as_uint(v.w), inv_scale);
  return ELEM == kE2M1 ? c0 | (c1 << 4) | (c2 << 8) | (c3 << 12)
                       : c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
}

// Block exponent from the bit pattern of amax (|x| bits, NaN/Inf compare
// above every finite value): floor(log2 amax) - emax clipped to [-127, 127].
template <int ELEM>
__device__ __forceinline__ int block_exponent(uint32_t a) {
  const int fl = a >= 0x00800000u ? (int)(a >> 23) - 127 : (31 - (int)__clz(a)) - 149;
  return min(max(fl - Fmt<ELEM>::kEmax, -127), 127);
}

__device__ __forceinline__ float scale_value(uint32_t byte) {
  // 2^(byte-127); byte 0 is the float32 subnormal 2^-127.
  return __uint_as_float(byte ? (byte << 23) : 0x00400000u);
}

// Nibble n (sign in bit 3) of an E2M1 code -> float bits, scaled.
__device__ __forceinline__ uint32_t decode_e2m1(uint32_t n, float scale) {
  const float mag = __uint_as_float((n & 7u) << 22) * 0x1p126f;
  return __float_as_uint(mag * scale) | ((n & 8u) << 28);
}

// Byte c of an E4M3 code -> float bits, scaled (NaN codes handled by caller).
__device__ __forceinline__ uint32_t decode_e4m3(uint32_t c, float scale) {
  const float mag = __uint_as_float((c & 0x7Fu) << 20) * 0x1p120f;
  const uint32_t v = __float_as_uint(mag * scale) | ((c & 0x80u) << 24);
  return (c & 0x7Fu) == 0x7Fu ? kNaN : v;
}

}  // namespace codec
}  // namespace mx
