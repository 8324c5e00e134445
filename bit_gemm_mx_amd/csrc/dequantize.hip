// MX dequantize: E2M1 / E4M3 codes + E8M0 scales -> float32, blocks along the
// last axis.  Table-free exact decode is in codec_common.h.
//
// Work mapping mirrors the quantize kernel: 8 lanes per block, each lane
// writes one 16-byte float4, so a wave's store instruction writes 1 KiB of
// contiguous memory; kUnroll independent blocks per lane and iteration.
#include "codec_common.h"

namespace mx {
namespace {

using namespace codec;

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
constexpr int kBlocksPerWaveIter = 8 * kUnroll;
typedef float f4v __attribute__((ext_vector_type(4)));

template <int ELEM>
__global__ void __launch_bounds__(kThreads)
dequantize_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                  float4* __restrict__ y, int64_t n_blocks) {
  const int lane = threadIdx.x & 63;
  const int sub = lane & 7;
  const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int64_t n_waves = ((int64_t)gridDim.x * kThreads) >> 6;
  const int64_t n_iter = (n_blocks + kBlocksPerWaveIter - 1) / kBlocksPerWaveIter;

  for (int64_t it = wave; it < n_iter; it += n_waves) {
    const int64_t blk0 = it * kBlocksPerWaveIter + (lane >> 3);
    uint32_t w[kUnroll];
    uint32_t sb[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t blk = blk0 + 8 * u;
      if (blk < n_blocks) {
        if (ELEM == kE2M1)
          w[u] = reinterpret_cast<const uint16_t*>(codes)[blk * 8 + sub];
        else
          w[u] = reinterpret_cast<const uint32_t*>(codes)[blk * 8 + sub];
        sb[u] = scales[blk];
      } else {
        w[u] = 0;
        sb[u] = 127;
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t blk = blk0 + 8 * u;
      const float s = scale_value(sb[u]);
      uint32_t o0, o1, o2, o3;
      if (ELEM == kE2M1) {
        o0 = decode_e2m1(w[u], s);
        o1 = decode_e2m1(w[u] >> 4, s);
        o2 = decode_e2m1(w[u] >> 8, s);
        o3 = decode_e2m1(w[u] >> 12, s);
      } else {
        o0 = decode_e4m3(w[u] & 0xFFu, s);
        o1 = decode_e4m3((w[u] >> 8) & 0xFFu, s);
        o2 = decode_e4m3((w[u] >> 16) & 0xFFu, s);
        o3 = decode_e4m3(w[u] >> 24, s);
      }
      if (sb[u] == 0xFFu) o0 = o1 = o2 = o3 = kNaN;
      if (blk < n_blocks) {
        // Output is written once and not read back by this kernel: a
        // non-temporal store (measured ~25% faster on the 8192x8192 stream).
        const f4v t = {__uint_as_float(o0), __uint_as_float(o1), __uint_as_float(o2),
                       __uint_as_float(o3)};
        __builtin_nontemporal_store(t, reinterpret_cast<f4v*>(&y[blk * 8 + sub]));
      }
    }
  }
}

int grid_for(int64_t n_blocks) {
  const int64_t iters = (n_blocks + kBlocksPerWaveIter - 1) / kBlocksPerWaveIter;
  int64_t wgs = (iters + kThreads / 64 - 1) / (kThreads / 64);
  const int64_t cap = 256 * 64;
  return (int)(wgs < cap ? wgs : cap);
}

}  // namespace

hipError_t launch_dequantize(const void* codes, const uint8_t* scales, float* y,
                             int64_t n_blocks, int elem, hipStream_t stream) {
  const int grid = grid_for(n_blocks);
  const uint8_t* c = static_cast<const uint8_t*>(codes);
  float4* y4 = reinterpret_cast<float4*>(y);
  if (elem == kE2M1)
    hipLaunchKernelGGL(dequantize_kernel<kE2M1>, dim3(grid), dim3(kThreads), 0, stream, c,
                       scales, y4, n_blocks);
  else
    hipLaunchKernelGGL(dequantize_kernel<kE4M3>, dim3(grid), dim3(kThreads), 0, stream, c,
                       scales, y4, n_blocks);
  return hipGetLastError();
}

}  // namespace mx
