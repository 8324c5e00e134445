// Memory floor of the decode-shaped block matmul launch (a benchmark
// reference, not part of libmx).
//
// Same grid as libmx's decode launch of a 16-row MXFP4 product: one
// workgroup of 8 waves per 16 columns of C, the K range of every row split
// over the 8 waves.  Each workgroup reads exactly the bytes the product
// reads -- its 16 rows of B^T codes and scales, and all of A's codes and
// scales -- with 16-byte loads, folds them into one word per lane so that
// no load can be dropped, and writes its 16 x 16 block of C.  No MFMA, no
// decode: its duration is what moving those bytes through that launch
// shape costs.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kWaves = 8;

// K = 4096 (the decode workload): per wave and row, K/8 codes = 256 bytes of
// a 2048-byte E2M1 row (16 chunks of 16 bytes) and 16 scale bytes (one
// chunk).  16 rows x 16 chunks = 4 chunks per lane, issued together.
__global__ void __launch_bounds__(64 * kWaves)
read_floor(const uint8_t* __restrict__ a, const uint8_t* __restrict__ sa,
           const uint8_t* __restrict__ bt, const uint8_t* __restrict__ sbt, float* __restrict__ c,
           int64_t M, int64_t N) {
  constexpr int64_t kRowBytes = 2048, kScaleRowBytes = 128, kSpan = kRowBytes / kWaves;
  __shared__ uint32_t red[kWaves][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  uint4 v[10];
#pragma unroll
  for (int j = 0; j < 4; ++j) {   // B^T codes: chunk i = 64 j + lane -> row i / 16, chunk i % 16
    const int i = 64 * j + lane;
    const int64_t row = min(n0 + i / 16, N - 1);
    v[j] = *reinterpret_cast<const uint4*>(bt + row * kRowBytes + wave * kSpan + 16 * (i % 16));
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {   // A codes, rows 0..M-1
    const int i = 64 * j + lane;
    const int64_t row = min((int64_t)(i / 16), M - 1);
    v[4 + j] = *reinterpret_cast<const uint4*>(a + row * kRowBytes + wave * kSpan + 16 * (i % 16));
  }
  {                               // scales: one 16-byte chunk per row and wave
    const int64_t rb = min(n0 + (lane & 15), N - 1), ra = min((int64_t)(lane & 15), M - 1);
    v[8] = *reinterpret_cast<const uint4*>(sbt + rb * kScaleRowBytes + 16 * wave);
    v[9] = *reinterpret_cast<const uint4*>(sa + ra * kScaleRowBytes + 16 * wave);
  }
  uint32_t acc = 0;
#pragma unroll
  for (int j = 0; j < 10; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  red[wave][lane] = acc;
  __syncthreads();
  for (int o = threadIdx.x; o < M * 16; o += 64 * kWaves) {
    uint32_t r = 0;
    for (int w = 0; w < kWaves; ++w) r ^= red[w][o & 63];
    const int64_t row = o / 16, col = n0 + (o % 16);
    if (col < N) c[row * N + col] = (float)(r & 0xFFFF);
  }
}

}  // namespace

// A: [M, K] E2M1 codes (K/2 bytes per row) and scales (K/32 per row); B^T:
// [N, K] likewise; C: [M, N] float32.  The loads are laid out for the decode
// workload: K must be 4096 and M at most 16.  Returns a hipError_t.
extern "C" int bench_read_floor(const void* a, const void* sa, const void* bt, const void* sbt,
                                float* c, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  if (!a || !sa || !bt || !sbt || !c || M < 1 || M > 16 || N < 1 || K != 4096)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(read_floor, dim3((unsigned)((N + 15) / 16)), dim3(64 * kWaves), 0, stream,
                     static_cast<const uint8_t*>(a), static_cast<const uint8_t*>(sa),
                     static_cast<const uint8_t*>(bt), static_cast<const uint8_t*>(sbt), c, M, N);
  return (int)hipGetLastError();
}
