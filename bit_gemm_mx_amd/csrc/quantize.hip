// MX quantize: float32 -> E2M1 / E4M3 codes + one E8M0 scale per 32 elements
// along the last axis.  Element rounding (fast hardware-convert path with an
// exact fallback at rounding midpoints) is in codec_common.h.
//
// Work mapping (HBM-bound stream, 4.53 B/element for E2M1):
//   * 8 lanes cover one 32-element block with one 16-byte load each, so a
//     wave's load instruction reads 1 KiB of contiguous memory;
//   * each lane keeps kUnroll loads in flight (4 KiB per wave per iteration);
//   * amax is an integer max over |x| bit patterns (exact, and any NaN/Inf
//     compares above every finite value) reduced over the 8 lanes with DPP.
#include "codec_common.h"

namespace mx {
namespace {

using namespace codec;

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
constexpr int kBlocksPerWaveIter = 8 * kUnroll;

// Max of v over each aligned group of 8 lanes.
__device__ __forceinline__ uint32_t max_over_8_lanes(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // lane ^ 1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // lane ^ 2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // 7 - lane
  return v;
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
      const int e = block_exponent<ELEM>(a);
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
