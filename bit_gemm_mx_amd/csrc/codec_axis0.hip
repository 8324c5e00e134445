// MX quantize / dequantize with blocks along axis 0 of a row-major
// [rows, cols] float32 matrix: block (i, c) = x[32i .. 32i+31, c].  The
// dialect page "A Dialect Is a Set of Co-Designed Decisions", section "The
// block axis": a block's scale must be constant along the reduction it
// multiplies, so a K x N matrix B is blocked along axis 0.
//
// Storage is block-major: codes [cols, rows/2] (E2M1, element 2k of a
// column's run in the low nibble of byte k) or [cols, rows] (E4M3), scales
// [cols, rows/32] -- the layout mx_quantize gives for the transposed matrix,
// which is the B^T operand layout of mx_block_matmul.  Element encode and
// decode are those of the last-axis kernels (codec_common.h).
//
// Work mapping: lane l of a wave owns column c0 + l and the wave walks kRun
// consecutive block-rows.  A row segment of 64 columns is 256 contiguous
// bytes, so every load (quantize) and store (dequantize) instruction on the
// float32 side is coalesced, and each lane holds its whole block in 32
// registers: amax, exponent and rounding need no cross-lane traffic.  Per
// lane, the codes of the kRun blocks are contiguous in memory (16 or 32 bytes
// each) and so are their kRun scale bytes.
#include "codec_common.h"

namespace mx {
namespace {

using namespace codec;

constexpr int kThreads = 256;
constexpr int kRun = 4;  // block-rows per wave (measured best of 4, 8, 16)

typedef uint32_t u4v __attribute__((ext_vector_type(4)));

// Wave task t -> (column strip, run of block-rows).  Consecutive tasks take
// adjacent strips of the same rows, so the waves in flight together read
// (quantize) or write (dequantize) whole rows of the float32 matrix: measured
// ~1.3x faster than walking down one strip.
struct Task {
  int64_t c;   // this lane's column
  int64_t ca;  // the column it addresses: c, or the last column for lanes past it
  int64_t i0;  // first block-row of the run
  bool live;   // column inside the matrix
};

__device__ __forceinline__ Task task_of(int64_t cols) {
  const int64_t t = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t n_strips = (cols + 63) / 64;
  const int64_t strip = t % n_strips, run = t / n_strips;
  Task k;
  k.c = strip * 64 + lane;
  k.i0 = run * kRun;
  k.live = k.c < cols;
  // Lanes past the last column load (and discard) the last column's data
  // instead of branching around their loads, so that every load of a block
  // is issued before the first one is waited for.
  k.ca = k.live ? k.c : cols - 1;
  return k;
}

__device__ __forceinline__ void load_block(float (&v)[32], const float* __restrict__ x,
                                           int64_t i, int64_t cols, const Task& k) {
  const float* p = x + 32 * i * cols + k.ca;
#pragma unroll
  for (int j = 0; j < 32; ++j) v[j] = __builtin_nontemporal_load(p + j * cols);
}

template <int ELEM>
struct Run {
  static constexpr int kBlockBytes = ELEM == kE2M1 ? 16 : 32;  // codes of one block
  static constexpr int kVecs = kBlockBytes / 16;
  u4v codes[kRun][kVecs];  // the run's codes, kRun x kBlockBytes contiguous bytes
  uint32_t bytes[kRun];    // the run's scale bytes
};

// Encode the run of block-rows [k.i0, k.i0 + run) of this lane's column.
// Block-rows are loaded kPf ahead of the one being encoded, into a ring of
// kPf + 1 register buffers indexed at compile time (measured: one block
// ahead 65 us, two 62.5 us, three no better, for the 8192x8192 E2M1 case).
template <int ELEM>
__device__ __forceinline__ void encode_run(Run<ELEM>& out, const float* __restrict__ x,
                                           int64_t cols, const Task& k, int run) {
  using F = Fmt<ELEM>;
  constexpr int kPf = 2;
  float vb[kPf + 1][32];
#pragma unroll
  for (int r = 0; r < kPf; ++r)
    if (r < run) load_block(vb[r], x, k.i0 + r, cols, k);
#pragma unroll
  for (int r = 0; r < kRun; ++r) {
    out.bytes[r] = 127u;
    if (r >= run) break;  // wave-uniform
    if (r + kPf < run) load_block(vb[(r + kPf) % (kPf + 1)], x, k.i0 + r + kPf, cols, k);
    const float* v = vb[r % (kPf + 1)];
    uint32_t amax = 0, low = 0xFFFFFFFFu;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const uint32_t b = __float_as_uint(v[j]);
      amax = max(amax, b & 0x7FFFFFFFu);
      low = min(low, b << F::kTieShift);
    }
    const int e = block_exponent<ELEM>(amax);
    const bool nonfinite = amax >= 0x7F800000u;
    out.bytes[r] = amax == 0 ? 127u : (nonfinite ? 0xFFu : (uint32_t)(e + 127));
    const float inv_scale = __uint_as_float((uint32_t)(127 - e) << 23);
    const float scale = __uint_as_float((uint32_t)max(e + 127, 1) << 23);
    const bool exact = k.live && (low == 0 || amax < 0x0D800000u);
    uint32_t w[8];  // codes of 4 consecutive elements each
    if (__ballot(exact) == 0) {
      const float top = ELEM == kE4M3 ? 448.0f * scale : 0.0f;
#pragma unroll
      for (int q = 0; q < 8; ++q)
        w[q] = convert4<ELEM>(make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]),
                              scale, top);
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q)
        w[q] = round4<ELEM>(make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]),
                            inv_scale);
    }
    if (nonfinite) {
#pragma unroll
      for (int q = 0; q < 8; ++q) w[q] = 0;
    }
    if (ELEM == kE2M1) {
      out.codes[r][0] = u4v{w[0] | (w[1] << 16), w[2] | (w[3] << 16), w[4] | (w[5] << 16),
                            w[6] | (w[7] << 16)};
    } else {
      out.codes[r][0] = u4v{w[0], w[1], w[2], w[3]};
      out.codes[r][Run<ELEM>::kVecs - 1] = u4v{w[4], w[5], w[6], w[7]};
    }
  }
}

// One wave per (64-column strip, run of kRun block-rows); each lane stores
// its run's codes (kRun x 16 or 32 contiguous bytes, half or whole cache
// lines) and scale bytes itself.  Any row count and scale alignment.
template <int ELEM>
__global__ void __launch_bounds__(kThreads)
quantize_axis0_kernel(const float* __restrict__ x, uint8_t* __restrict__ codes,
                      uint8_t* __restrict__ scales, int64_t rows, int64_t cols, int scale_vec) {
  const Task k = task_of(cols);
  const int64_t nbr = rows / 32;
  if (k.i0 >= nbr) return;  // wave-uniform: past the last run of the strip
  const int run = (int)min((int64_t)kRun, nbr - k.i0);
  const int64_t row_bytes = ELEM == kE2M1 ? rows / 2 : rows;
  constexpr int kBlockBytes = Run<ELEM>::kBlockBytes, kVecs = Run<ELEM>::kVecs;
  Run<ELEM> o;
  encode_run<ELEM>(o, x, cols, k, run);
  if (!k.live) return;
  uint8_t* crow = codes + k.c * row_bytes;
  uint8_t* srow = scales + k.c * nbr;
#pragma unroll
  for (int r = 0; r < kRun; ++r) {
    if (r < run) {
#pragma unroll
      for (int h = 0; h < kVecs; ++h)
        *reinterpret_cast<u4v*>(crow + (k.i0 + r) * kBlockBytes + 16 * h) = o.codes[r][h];
      if (!scale_vec) srow[k.i0 + r] = (uint8_t)o.bytes[r];
    }
  }
  // Whole runs with 4-byte aligned scale rows: one store of the run's bytes.
  if (scale_vec)
    *reinterpret_cast<uint32_t*>(srow + k.i0) =
        o.bytes[0] | (o.bytes[1] << 8) | (o.bytes[2] << 16) | (o.bytes[3] << 24);
}

// The eight waves of a workgroup take eight consecutive runs (32 block-rows)
// of the same 64-column strip, then store through LDS: each column's codes
// for the 32 block-rows are 512 (E2M1) or 1024 (E4M3) contiguous bytes and
// its 32 scale bytes are contiguous too, so every store instruction writes
// whole cache lines of a few columns instead of a 64-byte piece (and a
// 4-byte scale piece) of 64 columns 4 KiB apart.  With the stores removed
// the 8192x8192 E2M1 quantize reads its input in 46 us; the per-lane
// stores cost 16 us more, these 11 (four waves per workgroup and 256-byte
// pieces: 14; sixteen waves and 1 KiB pieces: 10).  Workgroups walk all
// strips of a row range before the next (bands of 4..32 strips down all
// rows measured 68-73 us).  Needs rows % 1024 == 0 and 16-byte aligned
// scale rows.
constexpr int kGroupRuns = 8;  // runs per workgroup
constexpr int kStagedThreads = 64 * kGroupRuns;

template <int ELEM>
__global__ void __launch_bounds__(kStagedThreads)
quantize_axis0_staged_kernel(const float* __restrict__ x, uint8_t* __restrict__ codes,
                             uint8_t* __restrict__ scales, int64_t rows, int64_t cols) {
  constexpr int kBlockBytes = Run<ELEM>::kBlockBytes, kVecs = Run<ELEM>::kVecs;
  constexpr int kColBytes = kGroupRuns * kRun * kBlockBytes;  // one column's codes here
  constexpr int kStride = kColBytes + 16;                     // padded LDS row
  __shared__ __attribute__((aligned(16))) uint8_t lds_codes[64 * kStride];
  __shared__ __attribute__((aligned(16))) uint32_t lds_scales[64 * kGroupRuns];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t n_strips = (cols + 63) / 64;
  const int64_t strip = blockIdx.x % n_strips, group = blockIdx.x / n_strips;
  Task k;
  k.c = strip * 64 + lane;
  k.live = k.c < cols;
  k.ca = k.live ? k.c : cols - 1;
  k.i0 = (group * kGroupRuns + wave) * kRun;
  Run<ELEM> o;
  encode_run<ELEM>(o, x, cols, k, kRun);
#pragma unroll
  for (int r = 0; r < kRun; ++r)
#pragma unroll
    for (int h = 0; h < kVecs; ++h)
      *reinterpret_cast<u4v*>(lds_codes + lane * kStride + (wave * kRun + r) * kBlockBytes +
                              16 * h) = o.codes[r][h];
  lds_scales[lane * kGroupRuns + wave] =
      o.bytes[0] | (o.bytes[1] << 8) | (o.bytes[2] << 16) | (o.bytes[3] << 24);
  __syncthreads();
  const int64_t row_bytes = ELEM == kE2M1 ? rows / 2 : rows;
  const int64_t c0 = strip * 64, b0 = group * kGroupRuns * kRun;  // first column, block-row
  constexpr int kChunks = kColBytes / 16;                         // 16-byte chunks per column
  constexpr int kColsPerPass = kStagedThreads / kChunks;
#pragma unroll
  for (int p = 0; p < 64 / kColsPerPass; ++p) {
    const int col = p * kColsPerPass + threadIdx.x / kChunks, ch = threadIdx.x % kChunks;
    if (c0 + col < cols)
      *reinterpret_cast<u4v*>(codes + (c0 + col) * row_bytes + b0 * kBlockBytes + 16 * ch) =
          *reinterpret_cast<const u4v*>(lds_codes + col * kStride + 16 * ch);
  }
  // 32 scale bytes per column: two 16-byte stores
  const int sc = threadIdx.x / 2, half = threadIdx.x & 1;
  if (threadIdx.x < 128 && c0 + sc < cols)
    *reinterpret_cast<u4v*>(scales + (c0 + sc) * (rows / 32) + b0 + 16 * half) =
        *reinterpret_cast<const u4v*>(lds_scales + sc * kGroupRuns + 4 * half);
}

template <int ELEM>
__global__ void __launch_bounds__(kThreads)
dequantize_axis0_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                        float* __restrict__ y, int64_t rows, int64_t cols, int scale_vec) {
  const Task k = task_of(cols);
  const int64_t nbr = rows / 32;
  if (k.i0 >= nbr) return;
  const int run = (int)min((int64_t)kRun, nbr - k.i0);
  const int64_t row_bytes = ELEM == kE2M1 ? rows / 2 : rows;
  constexpr int kBlockBytes = ELEM == kE2M1 ? 16 : 32;
  const uint8_t* crow = codes + k.ca * row_bytes;
  const uint8_t* srow = scales + k.ca * nbr;

  uint32_t sv = 0x7F7F7F7Fu;
  if (scale_vec) sv = *reinterpret_cast<const uint32_t*>(srow + k.i0);
  // The run's codes, loaded together up front: kRun x 16 or 32 contiguous
  // bytes per lane, half or whole cache lines.  Blocks past the run reload
  // the last block and go unused.
  constexpr int kVecs = kBlockBytes / 16;
  u4v cbuf[kRun][kVecs];
#pragma unroll
  for (int r = 0; r < kRun; ++r)
#pragma unroll
    for (int h = 0; h < kVecs; ++h)
      cbuf[r][h] = *reinterpret_cast<const u4v*>(crow + (k.i0 + min(r, run - 1)) * kBlockBytes +
                                                 16 * h);
#pragma unroll
  for (int r = 0; r < kRun; ++r) {
    if (r >= run) break;  // wave-uniform
    const int64_t i = k.i0 + r;
    const u4v d0 = cbuf[r][0], d1 = cbuf[r][kVecs - 1];
    const uint32_t byte =
        scale_vec ? ((sv >> (8 * (r & 3))) & 0xFFu) : srow[i];
    const float s = scale_value(byte);
    uint32_t o[32];
    if (ELEM == kE2M1) {
#pragma unroll
      for (int j = 0; j < 32; ++j) o[j] = decode_e2m1(d0[j >> 3] >> (4 * (j & 7)), s);
    } else {
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const uint32_t word = j < 16 ? d0[j >> 2] : d1[(j - 16) >> 2];
        o[j] = decode_e4m3((word >> (8 * (j & 3))) & 0xFFu, s);
      }
    }
    if (byte == 0xFFu) {
#pragma unroll
      for (int j = 0; j < 32; ++j) o[j] = kNaN;
    }
    if (k.live) {
#pragma unroll
      for (int j = 0; j < 32; ++j)
        __builtin_nontemporal_store(__uint_as_float(o[j]), &y[(32 * i + j) * cols + k.c]);
    }
  }
}

struct Launch {
  dim3 grid;
  int64_t n_runs;
  int scale_vec;
};

Launch plan(const uint8_t* scales, int64_t rows, int64_t cols) {
  const int64_t nbr = rows / 32;
  const int64_t n_runs = (nbr + kRun - 1) / kRun;
  const int64_t strips = (cols + 63) / 64;
  const int64_t waves = strips * n_runs;
  Launch l;
  l.grid = dim3((unsigned)((waves + kThreads / 64 - 1) / (kThreads / 64)));
  l.n_runs = n_runs;
  // Scale runs are stored / loaded as 4 bytes when every run is whole and
  // every column's scale row starts on a 4-byte boundary.
  l.scale_vec = (nbr % kRun == 0) && ((reinterpret_cast<uintptr_t>(scales) & 3) == 0);
  return l;
}

}  // namespace

hipError_t launch_quantize_axis0(const float* x, void* codes, uint8_t* scales, int64_t rows,
                                 int64_t cols, int elem, hipStream_t stream) {
  uint8_t* c = static_cast<uint8_t*>(codes);
  if (rows % (32 * kRun * kGroupRuns) == 0 && (reinterpret_cast<uintptr_t>(scales) & 15) == 0) {
    const int64_t groups = rows / (32 * kRun * kGroupRuns), strips = (cols + 63) / 64;
    if (groups * strips > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(groups * strips));
    if (elem == kE2M1)
      hipLaunchKernelGGL(quantize_axis0_staged_kernel<kE2M1>, grid, dim3(kStagedThreads), 0,
                         stream, x, c, scales, rows, cols);
    else
      hipLaunchKernelGGL(quantize_axis0_staged_kernel<kE4M3>, grid, dim3(kStagedThreads), 0,
                         stream, x, c, scales, rows, cols);
    return hipGetLastError();
  }
  const Launch l = plan(scales, rows, cols);
  if (l.grid.x == 0 || (int64_t)l.grid.x * (kThreads / 64) < ((cols + 63) / 64) * l.n_runs)
    return hipErrorInvalidValue;
  if (elem == kE2M1)
    hipLaunchKernelGGL(quantize_axis0_kernel<kE2M1>, l.grid, dim3(kThreads), 0, stream, x, c,
                       scales, rows, cols, l.scale_vec);
  else
    hipLaunchKernelGGL(quantize_axis0_kernel<kE4M3>, l.grid, dim3(kThreads), 0, stream, x, c,
                       scales, rows, cols, l.scale_vec);
  return hipGetLastError();
}

hipError_t launch_dequantize_axis0(const void* codes, const uint8_t* scales, float* y,
                                   int64_t rows, int64_t cols, int elem, hipStream_t stream) {
  const Launch l = plan(scales, rows, cols);
  if (l.grid.x == 0 || (int64_t)l.grid.x * (kThreads / 64) < ((cols + 63) / 64) * l.n_runs)
    return hipErrorInvalidValue;
  const uint8_t* c = static_cast<const uint8_t*>(codes);
  if (elem == kE2M1)
    hipLaunchKernelGGL(dequantize_axis0_kernel<kE2M1>, l.grid, dim3(kThreads), 0, stream, c,
                       scales, y, rows, cols, l.scale_vec);
  else
    hipLaunchKernelGGL(dequantize_axis0_kernel<kE4M3>, l.grid, dim3(kThreads), 0, stream, c,
                       scales, y, rows, cols, l.scale_vec);
  return hipGetLastError();
}

}  // namespace mx
