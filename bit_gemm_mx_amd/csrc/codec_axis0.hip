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
// Work mapping: lane l of a wave owns column c0 + l and the wave walks
// consecutive block-rows (kRun in the per-lane kernels, two per strip in the
// band kernel).  A row segment of 64 columns is 256 contiguous
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

// Encode one block held in this lane's registers: its codes (16 or 32
// bytes, element 0 first) and its scale byte.  `live` is false for lanes
// past the last column, which must not force the wave onto the exact path.
template <int ELEM>
__device__ __forceinline__ void encode_block(const float (&v)[32], bool live,
                                             u4v (&codes)[ELEM == kE2M1 ? 1 : 2],
                                             uint32_t& byte) {
  using F = Fmt<ELEM>;
  uint32_t amax = 0, low = 0xFFFFFFFFu;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const uint32_t b = __float_as_uint(v[j]);
    amax = max(amax, b & 0x7FFFFFFFu);
    low = min(low, b << F::kTieShift);
  }
  const int e = block_exponent<ELEM>(amax);
  const bool nonfinite = amax >= 0x7F800000u;
  byte = amax == 0 ? 127u : (nonfinite ? 0xFFu : (uint32_t)(e + 127));
  const float inv_scale = __uint_as_float((uint32_t)(127 - e) << 23);
  const float scale = __uint_as_float((uint32_t)max(e + 127, 1) << 23);
  const bool exact = live && (low == 0 || amax < 0x0D800000u);
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
  if constexpr (ELEM == kE2M1) {
    codes[0] = u4v{w[0] | (w[1] << 16), w[2] | (w[3] << 16), w[4] | (w[5] << 16),
                   w[6] | (w[7] << 16)};
  } else {
    codes[0] = u4v{w[0], w[1], w[2], w[3]};
    codes[1] = u4v{w[4], w[5], w[6], w[7]};
  }
}

// Encode the run of block-rows [k.i0, k.i0 + run) of this lane's column.
// Block-rows are loaded kPf ahead of the one being encoded, into a ring of
// kPf + 1 register buffers indexed at compile time (measured: one block
// ahead 65 us, two 62.5 us, three no better, for the 8192x8192 E2M1 case).
template <int ELEM>
__device__ __forceinline__ void encode_run(Run<ELEM>& out, const float* __restrict__ x,
                                           int64_t cols, const Task& k, int run) {
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
    encode_block<ELEM>(vb[r % (kPf + 1)], k.live, out.codes[r], out.bytes[r]);
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

// Band kernel.  A workgroup of 16 waves owns a band of 32 block-rows (1024
// rows) and, within it, kStrips consecutive 64-column strips, which it
// encodes one after the other: for each strip, wave w encodes block-rows 2w
// and 2w+1 of the band (lane l = column l of the strip) into LDS, and after
// a barrier the workgroup stores the strip -- each column's codes for the
// band (512 or 1024 contiguous bytes) and its 32 scale bytes, whole cache
// lines per store instruction.  The next strip's first block is loaded
// before that barrier, so its reads are in flight while the stores drain,
// and the two LDS buffers alternate by strip (a strip's encode never
// overwrites what the previous strip's stores still read: every thread
// passes the next barrier only after its own stores).  Tasks (band, strip)
// are numbered band-major and workgroup b takes tasks kStrips*b .. +kStrips-1,
// so the workgroups in flight write whole columns of codes and read every
// fourth 256-byte piece of all rows.  8192x8192 E2M1 on one box: 52.8 us
// (53.2 before the non-temporal code stores below) against 57.0 us for eight
// waves of four block-rows on one strip per workgroup (the quantize with its
// stores removed reads its input in
// 40.8 us; the stores, written contiguously instead of block-major, would
// take 53.9 us in that kernel -- it is the write stream mixed into the reads
// that costs, more than its layout).  Needs rows % 1024 == 0 and 16-byte
// aligned scale rows.
constexpr int kBandWaves = 16;
constexpr int kBandRun = 2;  // block-rows per wave and strip
constexpr int kBandBlocks = kBandWaves * kBandRun;
constexpr int kBandRows = 32 * kBandBlocks;
constexpr int kBandThreads = 64 * kBandWaves;
constexpr int kStrips = 4;   // strips per workgroup

template <int ELEM>
__global__ void __launch_bounds__(kBandThreads)
quantize_axis0_band_kernel(const float* __restrict__ x, uint8_t* __restrict__ codes,
                           uint8_t* __restrict__ scales, int64_t rows, int64_t cols) {
  constexpr int kBlockBytes = Run<ELEM>::kBlockBytes, kVecs = Run<ELEM>::kVecs;
  constexpr int kColBytes = kBandBlocks * kBlockBytes;  // one column's codes for the band
  constexpr int kStride = kColBytes + 16;               // padded LDS row
  __shared__ __attribute__((aligned(16))) uint8_t lds_codes[2][64 * kStride];
  __shared__ __attribute__((aligned(16))) uint8_t lds_sc[2][64 * kBandBlocks];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t n_strips = (cols + 63) / 64;
  const int64_t first = (int64_t)blockIdx.x * kStrips;
  // tasks of this workgroup (>= 1: the grid covers the tasks exactly)
  const int n_tasks = (int)min((int64_t)kStrips, (rows / kBandRows) * n_strips - first);
  const int64_t row_bytes = ELEM == kE2M1 ? rows / 2 : rows;
  // Block j of this wave's sequence: task first + j / kBandRun, block-row
  // kBandRun * wave + j % kBandRun of the task's band.  Lanes past the last
  // column load the last column (and discard it).
  auto load = [&](float (&v)[32], int j) {
    const int64_t task = first + j / kBandRun;
    const int64_t strip = task % n_strips, band = task / n_strips;
    const int64_t c = min(strip * 64 + lane, cols - 1);
    const int64_t i = band * kBandBlocks + kBandRun * wave + j % kBandRun;
    const float* p = x + 32 * i * cols + c;
#pragma unroll
    for (int q = 0; q < 32; ++q) v[q] = __builtin_nontemporal_load(p + q * cols);
  };
  float vb[2][32];
  load(vb[0], 0);
#pragma unroll
  for (int t = 0; t < kStrips; ++t) {
    if (t >= n_tasks) break;  // workgroup-uniform
    const int64_t task = first + t;
    const int64_t strip = task % n_strips, band = task / n_strips;
    const int64_t c0 = strip * 64;
    uint8_t* lc = lds_codes[t & 1];
    uint8_t* ls = lds_sc[t & 1];
#pragma unroll
    for (int r = 0; r < kBandRun; ++r) {
      const int j = t * kBandRun + r;
      if (j + 1 < n_tasks * kBandRun) load(vb[(j + 1) & 1], j + 1);
      u4v cv[kVecs];
      uint32_t byte;
      encode_block<ELEM>(vb[j & 1], c0 + lane < cols, cv, byte);
#pragma unroll
      for (int h = 0; h < kVecs; ++h)
        *reinterpret_cast<u4v*>(lc + lane * kStride + (kBandRun * wave + r) * kBlockBytes +
                                16 * h) = cv[h];
      ls[lane * kBandBlocks + kBandRun * wave + r] = (uint8_t)byte;
    }
    __syncthreads();
    const int64_t b0 = band * kBandBlocks;                 // first block-row of the band
    constexpr int kChunks = kColBytes / 16;                // 16-byte chunks per column
    constexpr int kColsPerPass = kBandThreads / kChunks;
    // Codes leave non-temporally: blocks along axis 0 are the weight side of
    // a product, read later by a matmul rather than right away, and the
    // streamed stores measured 54.0 -> 52.7 us (8192x8192 E2M1, rotating
    // outputs).  The 32-byte scale pieces keep ordinary stores: four
    // workgroups fill each 128-byte line, merged in L2 (non-temporal: 54.8).
#pragma unroll
    for (int p = 0; p < 64 / kColsPerPass; ++p) {
      const int col = p * kColsPerPass + threadIdx.x / kChunks, ch = threadIdx.x % kChunks;
      if (c0 + col < cols)
        __builtin_nontemporal_store(
            *reinterpret_cast<const u4v*>(lc + col * kStride + 16 * ch),
            reinterpret_cast<u4v*>(codes + (c0 + col) * row_bytes + b0 * kBlockBytes + 16 * ch));
    }
    // 32 scale bytes per column: two 16-byte stores
    const int sc = threadIdx.x / 2, half = threadIdx.x & 1;
    if (threadIdx.x < 128 && c0 + sc < cols)
      *reinterpret_cast<u4v*>(scales + (c0 + sc) * (rows / 32) + b0 + 16 * half) =
          *reinterpret_cast<const u4v*>(ls + sc * kBandBlocks + 16 * half);
  }
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

// Tile kernel for the dequantize.  A workgroup of 4 waves owns 4 adjacent
// 64-column strips (256 columns) and a run of 4 block-rows; for each
// block-row every wave decodes its strip's 32 x 64 values (lane = column)
// into LDS, and after a barrier the workgroup stores the 32 rows as 1 KiB
// pieces, 16 bytes per lane, where the per-lane kernel stores 256-byte row
// pieces 4 bytes per lane (32 store instructions per block instead of 8).
// 8192x8192 E2M1: 47.3 -> 45.5 us (2 or 4 strips per workgroup, one or two
// LDS tiles, the same; 8 or 16 strips 60-62 us, the LDS then holding one
// workgroup per CU).  Needs cols % 256 == 0, rows % 128 == 0 and 4-byte
// aligned scale rows.
constexpr int kTileStrips = 4;
constexpr int kTileRun = 4;  // block-rows per workgroup

template <int ELEM>
__global__ void __launch_bounds__(64 * kTileStrips)
dequantize_axis0_tile_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                             float* __restrict__ y, int64_t rows, int64_t cols) {
  typedef float f4v __attribute__((ext_vector_type(4)));
  constexpr int kBlockBytes = ELEM == kE2M1 ? 16 : 32, kVecs = kBlockBytes / 16;
  constexpr int kPad = 4;  // floats of padding per LDS row
  __shared__ __attribute__((aligned(16))) float tile[kTileStrips][32][64 + kPad];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t nbr = rows / 32, groups = cols / (64 * kTileStrips);
  const int64_t sg = blockIdx.x % groups, i0 = (blockIdx.x / groups) * kTileRun;
  const int64_t c = (sg * kTileStrips + wave) * 64 + lane;  // this lane's column
  const int64_t row_bytes = ELEM == kE2M1 ? rows / 2 : rows;
  const uint32_t sv = *reinterpret_cast<const uint32_t*>(scales + c * nbr + i0);
  u4v cb[kTileRun][kVecs];
#pragma unroll
  for (int r = 0; r < kTileRun; ++r)
#pragma unroll
    for (int h = 0; h < kVecs; ++h)
      cb[r][h] = *reinterpret_cast<const u4v*>(codes + c * row_bytes + (i0 + r) * kBlockBytes +
                                               16 * h);
#pragma unroll
  for (int r = 0; r < kTileRun; ++r) {
    const uint32_t byte = (sv >> (8 * r)) & 0xFFu;
    const float s = scale_value(byte);
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      uint32_t o;
      if (ELEM == kE2M1) {
        o = decode_e2m1(cb[r][0][j >> 3] >> (4 * (j & 7)), s);
      } else {
        const uint32_t word = j < 16 ? cb[r][0][j >> 2] : cb[r][kVecs - 1][(j - 16) >> 2];
        o = decode_e4m3((word >> (8 * (j & 3))) & 0xFFu, s);
      }
      tile[wave][j][lane] = __uint_as_float(byte == 0xFFu ? kNaN : o);
    }
    __syncthreads();
    // 32 rows x 1 KiB: wave w stores rows w, w + 4, ...; lane l the 16 bytes
    // at columns 4l .. 4l+3 of the workgroup's 256 (strip l / 16).
    float* yrow = y + 32 * (i0 + r) * cols + sg * 64 * kTileStrips + 4 * lane;
#pragma unroll
    for (int p = 0; p < 32 / kTileStrips; ++p) {
      const int row = kTileStrips * p + wave;
      const f4v v = *reinterpret_cast<const f4v*>(&tile[lane >> 4][row][4 * (lane & 15)]);
      __builtin_nontemporal_store(v, reinterpret_cast<f4v*>(yrow + row * cols));
    }
    __syncthreads();  // the tile is rewritten for the next block-row
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
  if (rows % kBandRows == 0 && (reinterpret_cast<uintptr_t>(scales) & 15) == 0) {
    const int64_t tasks = (rows / kBandRows) * ((cols + 63) / 64);
    const int64_t groups = (tasks + kStrips - 1) / kStrips;
    if (groups > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 grid((unsigned)groups);
    if (elem == kE2M1)
      hipLaunchKernelGGL(quantize_axis0_band_kernel<kE2M1>, grid, dim3(kBandThreads), 0, stream,
                         x, c, scales, rows, cols);
    else
      hipLaunchKernelGGL(quantize_axis0_band_kernel<kE4M3>, grid, dim3(kBandThreads), 0, stream,
                         x, c, scales, rows, cols);
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
  const uint8_t* c = static_cast<const uint8_t*>(codes);
  if (cols % (64 * kTileStrips) == 0 && rows % (32 * kTileRun) == 0 &&
      (reinterpret_cast<uintptr_t>(scales) & 3) == 0) {
    const int64_t wgs = (cols / (64 * kTileStrips)) * (rows / (32 * kTileRun));
    if (wgs > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (elem == kE2M1)
      hipLaunchKernelGGL(dequantize_axis0_tile_kernel<kE2M1>, dim3((unsigned)wgs),
                         dim3(64 * kTileStrips), 0, stream, c, scales, y, rows, cols);
    else
      hipLaunchKernelGGL(dequantize_axis0_tile_kernel<kE4M3>, dim3((unsigned)wgs),
                         dim3(64 * kTileStrips), 0, stream, c, scales, y, rows, cols);
    return hipGetLastError();
  }
  const Launch l = plan(scales, rows, cols);
  if (l.grid.x == 0 || (int64_t)l.grid.x * (kThreads / 64) < ((cols + 63) / 64) * l.n_runs)
    return hipErrorInvalidValue;
  if (elem == kE2M1)
    hipLaunchKernelGGL(dequantize_axis0_kernel<kE2M1>, l.grid, dim3(kThreads), 0, stream, c,
                       scales, y, rows, cols, l.scale_vec);
  else
    hipLaunchKernelGGL(dequantize_axis0_kernel<kE4M3>, l.grid, dim3(kThreads), 0, stream, c,
                       scales, y, rows, cols, l.scale_vec);
  return hipGetLastError();
}

}  // namespace mx
