// MX quantize: float32 -> E2M1 / E4M3 codes + one E8M0 scale per 32 elements.
//
// Semantics follow the "Bit Layout" page (mxfp4community.com), section
// "Reference encode and decode", with the exponent floor taken exactly:
//   amax -> e = clip(floor(log2 amax) - emax, -127, 127) -> byte e + 127,
//   y = |x| * 2^-e, nearest grid magnitude with ties to the smaller one,
//   saturation at the top of the grid, sign bit iff x < 0.
//
// Work mapping (HBM-bound stream, 4.53 B/element for E2M1):
//   * 8 lanes cover one 32-element block with one 16-byte load each, so a
//     wave's load instruction reads 1 KiB of contiguous memory;
//   * each lane keeps kUnroll loads in flight (4 KiB per wave per iteration);
//   * amax is an integer max over |x| bit patterns (exact, and any NaN/Inf
//     compares above every finite value) reduced over the 8 lanes with DPP.
//
// Rounding, fast path: gfx950's v_cvt_scalef32_pk_{fp4,fp8}_f32 compute the
// round-to-nearest-even code of x / s for a float scale s (checked on the
// hardware for every normal power-of-two scale), saturating for FP4 and
// overflowing to NaN for FP8 (so |x| is clamped to 448 * 2^e first).  Nearest
// with ties to the smaller magnitude differs from nearest-even only at exact
// midpoints, and a midpoint has at most 2 (E2M1) / 4 (E4M3) significant bits:
// its 21 / 19 low mantissa bits are zero.  -0.0 has them zero too.  So a wave
// takes the fast path unless one of its elements has those bits zero (or its
// block's scale is near the bottom of the range, where f32 subnormals and a
// subnormal scale appear); random data essentially never leaves it.
//
// Rounding, exact path: on the bit pattern of y, adding (half step - 1) and
// truncating the mantissa is round-to-nearest with ties down in the normal
// binades of the element format; the subnormal range (uniform spacing) uses
// ceil(y / spacing - 1/2), which also rounds ties down.
#include "mx_internal.h"

namespace mx {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
constexpr int kBlocksPerWaveIter = 8 * kUnroll;

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

// Max of v over each aligned group of 8 lanes.
__device__ __forceinline__ uint32_t max_over_8_lanes(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // lane ^ 1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // lane ^ 2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // 7 - lane
  return v;
}

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

template <int ELEM>
__global__ void __launch_bounds__(kThreads)
quantize_kernel(const float4* __restrict__ x, uint8_t* __restrict__ codes,
                uint8_t* __restrict__ scales, int64_t n_blocks) {
  using F = Fmt<ELEM>;
  const int lane = threadIdx.x & 63;
  const int sub = lane & 7;  // which 16-byte quarter-row of the block
  const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int64_t n_waves = ((int64_t)gridDim.x * kThreads) >> 6;
  const int64_t n_iter = (n_blocks + kBlocksPerWaveIter - 1) / kBlocksPerWaveIter;

  for (int64_t it = wave; it < n_iter; it += n_waves) {
    const int64_t blk0 = it * kBlocksPerWaveIter + (lane >> 3);
    float4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t blk = blk0 + 8 * u;
      if (blk < n_blocks) {
        // Each input byte is read once: a non-temporal load does not displace
        // useful cache lines.
        const f4v t = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(&x[blk * 8 + sub]));
        v[u] = make_float4(t[0], t[1], t[2], t[3]);
      } else {
        v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    uint32_t amax[kUnroll];
    uint32_t low = 0xFFFFFFFFu;  // min over elements of their low mantissa bits
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t b0 = __float_as_uint(v[u].x), b1 = __float_as_uint(v[u].y);
      const uint32_t b2 = __float_as_uint(v[u].z), b3 = __float_as_uint(v[u].w);
      amax[u] = max(max(b0 & 0x7FFFFFFFu, b1 & 0x7FFFFFFFu), max(b2 & 0x7FFFFFFFu, b3 & 0x7FFFFFFFu));
      low = min(low, min(min(b0 << F::kTieShift, b1 << F::kTieShift),
                         min(b2 << F::kTieShift, b3 << F::kTieShift)));
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) amax[u] = max_over_8_lanes(amax[u]);

    float inv_scale[kUnroll], scale[kUnroll];
    uint32_t byte[kUnroll];
    bool nonfinite[kUnroll];
    bool exact = low == 0;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      // floor(log2 amax) from the bit pattern (subnormals via the leading bit).
      const uint32_t a = amax[u];
      const int fl = a >= 0x00800000u ? (int)(a >> 23) - 127 : (31 - (int)__clz(a)) - 149;
      const int e = min(max(fl - F::kEmax, -127), 127);
      inv_scale[u] = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e, normal
      nonfinite[u] = a >= 0x7F800000u;
      byte[u] = a == 0 ? 127u : (nonfinite[u] ? 0xFFu : (uint32_t)(e + 127));
      // 2^e itself, for the convert; blocks below amax 2^-100 (and all-zero
      // blocks) take the exact path.
      scale[u] = __uint_as_float((uint32_t)max(e + 127, 1) << 23);
      exact |= a < 0x0D800000u;
    }

    if (__ballot(exact) == 0) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t blk = blk0 + 8 * u;
        const float top = ELEM == kE4M3 ? 448.0f * scale[u] : 0.0f;
        uint32_t w = convert4<ELEM>(v[u], scale[u], top);
        w = nonfinite[u] ? 0u : w;
        if (blk < n_blocks) {
          if (ELEM == kE2M1)
            reinterpret_cast<uint16_t*>(codes)[blk * 8 + sub] = (uint16_t)w;
          else
            reinterpret_cast<uint32_t*>(codes)[blk * 8 + sub] = w;
          if (sub == 0) scales[blk] = (uint8_t)byte[u];
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t blk = blk0 + 8 * u;
        uint32_t w = round4<ELEM>(v[u], inv_scale[u]);
        w = nonfinite[u] ? 0u : w;
        if (blk < n_blocks) {
          if (ELEM == kE2M1)
            reinterpret_cast<uint16_t*>(codes)[blk * 8 + sub] = (uint16_t)w;
          else
            reinterpret_cast<uint32_t*>(codes)[blk * 8 + sub] = w;
          if (sub == 0) scales[blk] = (uint8_t)byte[u];
        }
      }
    }
  }
}

int grid_for(int64_t n_blocks) {
  const int64_t iters = (n_blocks + kBlocksPerWaveIter - 1) / kBlocksPerWaveIter;
  const int64_t waves_per_wg = kThreads / 64;
  int64_t wgs = (iters + waves_per_wg - 1) / waves_per_wg;
  // Enough workgroups to fill 256 CUs many times over (measured best for the
  // 8192x8192 stream); the grid-stride loop covers the rest.
  const int64_t cap = 256 * 64;
  return (int)(wgs < cap ? wgs : cap);
}

}  // namespace

hipError_t launch_quantize(const float* x, void* codes, uint8_t* scales, int64_t n_blocks,
                           int elem, hipStream_t stream) {
  const int grid = grid_for(n_blocks);
  const float4* x4 = reinterpret_cast<const float4*>(x);
  uint8_t* c = static_cast<uint8_t*>(codes);
  if (elem == kE2M1)
    hipLaunchKernelGGL(quantize_kernel<kE2M1>, dim3(grid), dim3(kThreads), 0, stream, x4, c,
                       scales, n_blocks);
  else
    hipLaunchKernelGGL(quantize_kernel<kE4M3>, dim3(grid), dim3(kThreads), 0, stream, x4, c,
                       scales, n_blocks);
  return hipGetLastError();
}

}  // namespace mx
