// fold_scale: multiply a block-scaled tensor by 2^j through its E8M0 scale
// bytes alone.  The dialect page "A Dialect Is a Set of Co-Designed
// Decisions", section "The four ops" (fold_scale handles a scalar multiply of
// a block-scaled value without touching its elements; exact for powers of
// two), and the "Bit Layout" page, section "The E8M0 shared scale" (byte s
// stands for 2^(s-127); 0xFF is NaN).  Byte s becomes s + j when s != 0xFF
// and 0 <= s + j <= 254; otherwise no E8M0 byte holds the product and the
// block becomes NaN (0xFF).
//
// A byte stream: 16 bytes per lane in the aligned body, bytes one by one in
// the unaligned head and the tail.
#include "mx_internal.h"

namespace mx {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t fold_byte(uint32_t s, int j) {
  const int t = (int)s + j;
  return (s == 0xFFu || t < 0 || t > 254) ? 0xFFu : (uint32_t)t;
}

__device__ __forceinline__ uint32_t fold_word(uint32_t w, int j) {
  return fold_byte(w & 0xFFu, j) | (fold_byte((w >> 8) & 0xFFu, j) << 8) |
         (fold_byte((w >> 16) & 0xFFu, j) << 16) | (fold_byte(w >> 24, j) << 24);
}

__global__ void __launch_bounds__(kThreads)
fold_scale_kernel(uint8_t* __restrict__ s, int64_t head, int64_t n_vec, int64_t tail, int j) {
  const int64_t tid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  if (tid < head) s[tid] = (uint8_t)fold_byte(s[tid], j);
  uint4* body = reinterpret_cast<uint4*>(s + head);
  for (int64_t v = tid; v < n_vec; v += stride) {
    uint4 w = body[v];
    w.x = fold_word(w.x, j);
    w.y = fold_word(w.y, j);
    w.z = fold_word(w.z, j);
    w.w = fold_word(w.w, j);
    body[v] = w;
  }
  if (tid < tail) {
    uint8_t* t = s + head + 16 * n_vec;
    t[tid] = (uint8_t)fold_byte(t[tid], j);
  }
}

}  // namespace

hipError_t launch_fold_scale(uint8_t* scales, int64_t n, int j, hipStream_t stream) {
  // Every result is 0xFF once |j| > 254; clamping j keeps the arithmetic in int.
  j = j < -255 ? -255 : (j > 255 ? 255 : j);
  const int64_t head = min(n, (int64_t)((16 - (reinterpret_cast<uintptr_t>(scales) & 15)) & 15));
  const int64_t n_vec = (n - head) / 16;
  const int64_t tail = n - head - 16 * n_vec;
  int64_t blocks = (n_vec + kThreads - 1) / kThreads;
  blocks = blocks < 1 ? 1 : (blocks > 4096 ? 4096 : blocks);
  hipLaunchKernelGGL(fold_scale_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                     scales, head, n_vec, tail, j);
  return hipGetLastError();
}

}  // namespace mx
