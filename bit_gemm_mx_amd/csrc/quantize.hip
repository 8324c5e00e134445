// MX quantize: float32 -> E2M1 / E4M3 codes + one E8M0 scale per 32 elements
// along the last axis.  Element rounding (fast hardware-convert path with an
// exact fallback at rounding midpoints) is in codec_common.h.
//
// Work mapping (HBM-bound stream, 4.53 B/element for E2M1):
//   * 8 lanes cover one 32-element block with one 16-byte load each, so a
//     wave's load instruction reads 1 KiB of contiguous memory;
//   * each lane keeps kUnroll loads in flight (4 KiB per wave per iteration);
//   * amax is an integer max over |x| bit patterns (exact, and any NaN/Inf
//     compares above every finite value) reduced over the 8 lanes with DPP;
//   * a wave's codes and scale bytes for its 32 blocks go through its own
//     LDS slot and leave as 16-byte stores (512 or 1024 bytes of codes and
//     32 scale bytes per wave) instead of 2- or 4-byte stores per lane and
//     single scale bytes.  The read stream is what a quantize is made of
//     (4 of its 4.53 bytes per element) and the write stream mixed into it
//     costs more than its bytes; fewer, wider stores cost less.  Measured on
//     the 8192x8192 E2M1 case: 50.0 -> 47.7 us with workgroups of 8 waves
//     (48.9 us with 4 waves, 52.4 with 16); with its stores removed the
//     kernel reads its input in 38.6 us.
#include "codec_common.h"

namespace mx {
namespace {

using namespace codec;

constexpr int kThreads = 512;
constexpr int kUnroll = 4;
constexpr int kBlocksPerWaveIter = 8 * kUnroll;

typedef uint32_t u4v __attribute__((ext_vector_type(4)));

// Max of v over each aligned group of 8 lanes.
__device__ __forceinline__ uint32_t max_over_8_lanes(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // lane ^ 1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // lane ^ 2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // 7 - lane
  return v;
}

// STAGED: every wave iteration is whole (n_blocks a multiple of 32) and the
// scales are 16-byte aligned, so codes and scales leave through LDS as
// 16-byte stores; otherwise each lane stores its own codes and scale bytes.
template <int ELEM, bool STAGED>
__global__ void __launch_bounds__(kThreads)
quantize_kernel(const float4* __restrict__ x, uint8_t* __restrict__ codes,
                uint8_t* __restrict__ scales, int64_t n_blocks) {
  using F = Fmt<ELEM>;
  constexpr int kWaveCodes = kBlocksPerWaveIter * (ELEM == kE2M1 ? 16 : 32);  // bytes
  // Per wave: its codes, then its scale bytes.
  __shared__ __attribute__((aligned(16))) uint8_t stage[kThreads / 64][kWaveCodes +
                                                                       kBlocksPerWaveIter];
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
      // Each input byte is read once: a non-temporal load does not displace
      // useful cache lines.  Staged iterations are whole: no branch around
      // the loads (with one, the compiler issues each load behind its own
      // exec-mask branch).
      if (STAGED || blk < n_blocks) {
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

    uint32_t w[kUnroll];  // this lane's codes of its 4 elements of each block
    if (__ballot(exact) == 0) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const float top = ELEM == kE4M3 ? 448.0f * scale[u] : 0.0f;
        w[u] = nonfinite[u] ? 0u : convert4<ELEM>(v[u], scale[u], top);
      }
    } else {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) w[u] = nonfinite[u] ? 0u : round4<ELEM>(v[u], inv_scale[u]);
    }

    if constexpr (STAGED) {
      // Stage the wave's codes and scale bytes in its LDS slot (block b =
      // 8u + lane / 8 of the iteration, lane quarter sub), then store them
      // as 16-byte pieces.
      uint8_t* l = stage[threadIdx.x >> 6];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int b = 8 * u + (lane >> 3);
        if (ELEM == kE2M1)
          reinterpret_cast<uint16_t*>(l)[b * 8 + sub] = (uint16_t)w[u];
        else
          reinterpret_cast<uint32_t*>(l)[b * 8 + sub] = w[u];
        if (sub == 0) l[kWaveCodes + b] = (uint8_t)byte[u];
      }
      // LDS accesses of one wave complete in order; the wait also keeps the
      // compiler from moving the reads above the writes of other lanes.
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      constexpr int kPieces = kWaveCodes / 16;  // 32 or 64 code pieces, then 2 scale pieces
#pragma unroll
      for (int p = 0; p < (kPieces + 2 + 63) / 64; ++p) {
        const int idx = 64 * p + lane;
        if (idx < kPieces)
          reinterpret_cast<u4v*>(codes + it * kWaveCodes)[idx] =
              reinterpret_cast<const u4v*>(l)[idx];
        else if (idx < kPieces + 2)
          reinterpret_cast<u4v*>(scales + it * kBlocksPerWaveIter)[idx - kPieces] =
              reinterpret_cast<const u4v*>(l + kWaveCodes)[idx - kPieces];
      }
    } else {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t blk = blk0 + 8 * u;
        if (blk < n_blocks) {
          if (ELEM == kE2M1)
            reinterpret_cast<uint16_t*>(codes)[blk * 8 + sub] = (uint16_t)w[u];
          else
            reinterpret_cast<uint32_t*>(codes)[blk * 8 + sub] = w[u];
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
  // Enough workgroups to fill 256 CUs many times over (one iteration per wave
  // for the 8192x8192 stream); the grid-stride loop covers the rest.
  const int64_t cap = 256 * 32;
  return (int)(wgs < cap ? wgs : cap);
}

}  // namespace

hipError_t launch_quantize(const float* x, void* codes, uint8_t* scales, int64_t n_blocks,
                           int elem, hipStream_t stream) {
  uint8_t* c = static_cast<uint8_t*>(codes);
  const int64_t code_bytes = elem == kE2M1 ? 16 : 32;  // per block
  // Whole wave iterations with 16-byte aligned scales take the staged
  // stores; a ragged tail (n_blocks % 32 blocks) or unaligned scales the
  // per-lane ones, in a launch of their own.
  const int64_t n_main =
      (reinterpret_cast<uintptr_t>(scales) & 15) == 0 ? n_blocks / kBlocksPerWaveIter *
                                                            kBlocksPerWaveIter : 0;
  if (n_main > 0) {
    const float4* x4 = reinterpret_cast<const float4*>(x);
    if (elem == kE2M1)
      hipLaunchKernelGGL((quantize_kernel<kE2M1, true>), dim3(grid_for(n_main)), dim3(kThreads),
                         0, stream, x4, c, scales, n_main);
    else
      hipLaunchKernelGGL((quantize_kernel<kE4M3, true>), dim3(grid_for(n_main)), dim3(kThreads),
                         0, stream, x4, c, scales, n_main);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t rest = n_blocks - n_main;
  if (rest > 0) {
    const float4* x4 = reinterpret_cast<const float4*>(x + n_main * 32);
    if (elem == kE2M1)
      hipLaunchKernelGGL((quantize_kernel<kE2M1, false>), dim3(grid_for(rest)), dim3(kThreads),
                         0, stream, x4, c + n_main * code_bytes, scales + n_main, rest);
    else
      hipLaunchKernelGGL((quantize_kernel<kE4M3, false>), dim3(grid_for(rest)), dim3(kThreads),
                         0, stream, x4, c + n_main * code_bytes, scales + n_main, rest);
  }
  return hipGetLastError();
}

}  // namespace mx
