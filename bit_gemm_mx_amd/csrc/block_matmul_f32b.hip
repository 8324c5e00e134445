// MX block matmul with an ordinary float32 B: C[M,N] (+)= A[M,K] . B[K,N],
// A block-scaled along K (codes + E8M0 scales), B row-major float32 [K, N].
// This is block_matmul as the dialect page "A Dialect Is a Set of
// Co-Designed Decisions" states its first version (section "The four ops":
// a block-scaled A of shape MxK, an ordinary f32 B of shape KxN, C += A.B;
// section "The accumulator operand": C is updated in place).
//
// Arithmetic: A's elements are decoded exactly (grid value x 2^(byte-127),
// by the hardware's scaled converts) and multiplied with B on the fp32 matrix cores
// (v_mfma_f32_16x16x4_f32).  Each 32-element block of K is summed into a
// fresh accumulator P, blocks are summed into G in groups of 16, and groups
// into T -- each partial sum spans at most 32 products, 16 blocks or K/512
// groups, so the fp32 rounding error stays near 64 ulp of sum |a b| at
// K = 8192 instead of growing with K.  A NaN scale byte or E4M3 NaN code makes
// the outputs of its row NaN.
//
// MFMA layout (16x16x4 f32): lane l supplies A[l % 16][l / 16] and
// B[l / 16][l % 16] of the 16x4 / 4x16 operand step and holds
// C[4 (l / 16) + r][l % 16], r = 0..3.  Operands come straight from global
// memory into registers: a lane loads its quarter of the code block of its A
// row (the 4 lanes of a row read the block's 16 or 32 contiguous bytes) and
// 8 of B's rows for its column, 64 contiguous bytes per 16 lanes; loads run
// one batch of blocks ahead of the MFMAs.  No LDS staging: at the fp32 matrix
// rate the operand traffic per MFMA is small.
//
// Launch shapes: a 128x64 tile per workgroup (4 waves of 4x2 MFMA tiles,
// whole K each) when that gives at least one workgroup per CU; otherwise a
// 16x16 tile per workgroup whose 16 waves split K (four waves per SIMD hide
// each other's load and MFMA latencies) and add their partial sums in LDS in
// a fixed order (so results do not depend on timing).  The K-split shape
// streams its operands through LDS in 16-byte pieces when K % 256 == 0,
// N % 4 == 0 and B is 16-byte aligned (block_matmul_f32b_stream), else it
// loads them element-wise (block_matmul_f32b_kernel).
#include "codec_common.h"

namespace mx {
namespace {

using namespace codec;

typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u4v __attribute__((ext_vector_type(4)));


// Raw operand data of one 32-element block of K for one 16-row tile of A and
// one 16-column tile of B, as loaded.  Lane group q (= lane / 16) owns the
// eight consecutive elements 8q .. 8q+7 of the block: K step s of the MFMA
// takes element 8q + s from lane group q, for A and for B alike.  So a lane
// loads one dword (E2M1) or two (E4M3) of its A row's code block and the
// block's scale byte, and B's rows 8q .. 8q+7 of the block for its column.
struct RawA {
  uint32_t w0, w1;  // w1 used by E4M3 only
  uint32_t byte;
};

// Loads are issued unconditionally: rows past M and columns past N address
// the last row / column, and blocks past the end address the last block, so
// a batch of loads never sits behind a branch.  Output row i of an MFMA tile
// depends only on A row i and output column j only on B column j, so what
// such lanes load only reaches outputs that are never stored.
template <int ELEM>
__device__ __forceinline__ void load_a(RawA& r, const uint8_t* __restrict__ codes,
                                       const uint8_t* __restrict__ scales, int64_t row, int64_t j,
                                       int64_t kb, int q) {
  r.byte = scales[row * kb + j];
  if (ELEM == kE2M1) {
    r.w0 = *reinterpret_cast<const uint32_t*>(codes + row * (kb * 16) + j * 16 + 4 * q);
  } else {
    const uint2 v = *reinterpret_cast<const uint2*>(codes + row * (kb * 32) + j * 32 + 8 * q);
    r.w0 = v.x;
    r.w1 = v.y;
  }
}

__device__ __forceinline__ void load_b(float (&v)[8], const float* __restrict__ b, int64_t col,
                                       int64_t N, int64_t j, int q) {
  const float* p = b + (32 * j + 8 * q) * N + col;
#pragma unroll
  for (int s = 0; s < 8; ++s) v[s] = p[s * N];
}

typedef float v2f __attribute__((ext_vector_type(2)));

// Decoded, scaled A values of K steps s = 0..7 (elements 8q + s of the
// block).  gfx950's scaled converts give code value x 2^(byte-127) exactly
// for every code and scale byte (checked exhaustively on the hardware,
// subnormal results and the subnormal scale 2^-127 included); a 0xFF byte is
// passed as a NaN scale, so the whole block decodes to NaN.
template <int ELEM>
__device__ __forceinline__ void decode_a(float (&v)[8], const RawA& r) {
  const float sc = r.byte == 0xFFu ? __uint_as_float(kNaN) : scale_value(r.byte);
  if (ELEM == kE2M1) {
    const v2f p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r.w0, sc, 0);
    const v2f p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r.w0, sc, 1);
    const v2f p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r.w0, sc, 2);
    const v2f p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r.w0, sc, 3);
    v[0] = p0.x; v[1] = p0.y; v[2] = p1.x; v[3] = p1.y;
    v[4] = p2.x; v[5] = p2.y; v[6] = p3.x; v[7] = p3.y;
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t word = h ? r.w1 : r.w0;
      const v2f lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(word, sc, false);
      const v2f hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(word, sc, true);
      v[4 * h] = lo.x;
      v[4 * h + 1] = lo.y;
      v[4 * h + 2] = hi.x;
      v[4 * h + 3] = hi.y;
    }
  }
}

// TI x TJ tiles of 16x16 per wave.  SPLIT = 1: 4 waves tile the
// workgroup's (2 TI x 16) x (2 TJ x 16) block of C, each over all of K.
// SPLIT > 1: SPLIT waves share one (TI x 16) x (TJ x 16) block and split K.
// U blocks of K are loaded per batch, one batch ahead of the MFMAs.
template <int SPLIT>
constexpr int f32b_threads() { return 64 * (SPLIT == 1 ? 4 : SPLIT); }

template <int ELEM, int SPLIT, int TI, int TJ, int U>
__global__ void __launch_bounds__(f32b_threads<SPLIT>())
block_matmul_f32b_kernel(const uint8_t* __restrict__ a, const uint8_t* __restrict__ sa,
                         const float* __restrict__ b, float* __restrict__ c, int64_t M, int64_t N,
                         int64_t K, int accumulate, int tiles_n) {
  constexpr int WM = SPLIT == 1 ? 2 : 1, WN = SPLIT == 1 ? 2 : 1;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r16 = lane & 15, q = lane >> 4;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int wm = SPLIT == 1 ? (w >> 1) : 0, wn = SPLIT == 1 ? (w & 1) : 0;
  const int64_t m0 = (int64_t)tm * (WM * TI * 16) + wm * (TI * 16);
  const int64_t n0 = (int64_t)tn * (WN * TJ * 16) + wn * (TJ * 16);
  const int64_t kb = K / 32;
  const int64_t jb = SPLIT == 1 ? 0 : (kb * w) / SPLIT;
  const int64_t je = SPLIT == 1 ? kb : (kb * (w + 1)) / SPLIT;

  int64_t arow[TI], bcol[TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i) arow[i] = min(m0 + 16 * i + r16, M - 1);
#pragma unroll
  for (int t = 0; t < TJ; ++t) bcol[t] = min(n0 + 16 * t + r16, N - 1);

  v4f T[TI][TJ], G[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int t = 0; t < TJ; ++t) T[i][t] = G[i][t] = v4f{0.f, 0.f, 0.f, 0.f};

  RawA ra[2][U][TI];
  float rb[2][U][TJ][8];
  auto load_batch = [&](const int slot, int64_t j0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = min(j0 + u, je - 1);
#pragma unroll
      for (int i = 0; i < TI; ++i) load_a<ELEM>(ra[slot][u][i], a, sa, arow[i], j, kb, q);
#pragma unroll
      for (int t = 0; t < TJ; ++t) load_b(rb[slot][u][t], b, bcol[t], N, j, q);
    }
  };
  auto compute_batch = [&](const int slot, int64_t j0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = j0 + u;
      if (j >= je) break;  // wave-uniform
      float av[TI][8];
#pragma unroll
      for (int i = 0; i < TI; ++i) decode_a<ELEM>(av[i], ra[slot][u][i]);
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int t = 0; t < TJ; ++t) {
          const float* bv = rb[slot][u][t];
          v4f P = __builtin_amdgcn_mfma_f32_16x16x4f32(av[i][0], bv[0],
                                                       v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
          for (int s = 1; s < 8; ++s)
            P = __builtin_amdgcn_mfma_f32_16x16x4f32(av[i][s], bv[s], P, 0, 0, 0);
          G[i][t] += P;
        }
      if (((j - jb) & 15) == 15) {
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int t = 0; t < TJ; ++t) {
            T[i][t] += G[i][t];
            G[i][t] = v4f{0.f, 0.f, 0.f, 0.f};
          }
      }
    }
  };

  // Two register slots, alternated with compile-time indices; loads past the
  // end reload the last block and go unused.
  if (jb < je) {
    load_batch(0, jb);
    for (int64_t j0 = jb; j0 < je; j0 += 2 * U) {
      load_batch(1, j0 + U);
      compute_batch(0, j0);
      if (j0 + U >= je) break;  // wave-uniform
      load_batch(0, j0 + 2 * U);
      compute_batch(1, j0 + U);
    }
  }
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int t = 0; t < TJ; ++t) T[i][t] += G[i][t];

  if (SPLIT > 1) {
    // Partial sums of the SPLIT K ranges, added in wave order.
    __shared__ v4f red[SPLIT][TI][TJ][64];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int t = 0; t < TJ; ++t) red[w][i][t][lane] = T[i][t];
    __syncthreads();
    if (w != 0) return;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int t = 0; t < TJ; ++t) {
        v4f s = red[0][i][t][lane];
#pragma unroll
        for (int x = 1; x < SPLIT; ++x) s += red[x][i][t][lane];
        T[i][t] = s;
      }
  }
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int t = 0; t < TJ; ++t) {
      const int64_t col = n0 + 16 * t + r16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = m0 + 16 * i + 4 * q + r;
        if (row < M && col < N) {
          float v = T[i][t][r];
          if (accumulate) v += c[row * N + col];
          c[row * N + col] = v;
        }
      }
    }
}

// Streamed variant of the K-split shape for few output tiles (the decode
// product): one 16x16 tile of C per workgroup, 16 waves, each owning whole
// units of 256 K (8 blocks).  Measured on the 4096x4096 . 4096x16 decode
// shape: 9.1 us against 12.8 us for the plain K-split kernel; the remaining
// time is the fp32 MFMAs (~3.8 us per SIMD at one unit per wave) plus a
// fixed ~2.9 us of launch, first-load latency and the final reduction.  The plain K-split kernel above is bound by its
// vector memory path: per 32-K step a wave issues a dword load that touches
// 16 A rows, a byte load for 16 scales and eight dword loads of B (~64 cache
// lines).  Here a unit's operands arrive in whole 16-byte pieces:
//  * A: lane (r, q) loads the 32 (E2M1) or 64 (E4M3) contiguous code bytes
//    of row r that hold the unit's blocks 2q and 2q + 1, and their two scale
//    bytes.  Lane group q thus supplies the unit's K values 64q .. 64q + 63,
//    in order, to the unit's 64 MFMAs: which K a lane group supplies is free
//    as long as A and B agree, and A's values arrive decoded and scaled, so
//    one MFMA may take different blocks from different lane groups.
//  * B: MFMA t of the unit needs rows k0 + 64q + t of the tile's 16 columns
//    in lane group q.  The unit is taken in quarters of 16 MFMAs; a quarter's
//    4 x 16 rows (four 1 KiB row runs, one per lane group) are copied by
//    buffer loads that write LDS directly into one of the wave's two stage
//    buffers, and each lane then reads its column of a row from LDS.  The
//    next quarter's copy is in flight while a quarter is multiplied.
// Partial sums keep the plain kernel's structure: a fresh accumulator P per
// 8 MFMAs (32 products), P added into G, G into T every 16 P.
// Requires K % 256 == 0 and N % 4 == 0 (the launcher checks); rows past M and
// column groups past N read the last valid ones and reach only outputs that
// are not stored.
constexpr int kStreamWaves = 16;
constexpr int kRunBytes = 1024 + 64;   // 16 rows x 64 B; + 64 puts the 4 runs 16 banks apart
constexpr int kStageBytes = 4 * kRunBytes;
constexpr int kWaveLds = 2 * kStageBytes;
constexpr int kLgkm0 = 0xC07F;         // s_waitcnt lgkmcnt(0), other counters untouched

__device__ __forceinline__ constexpr int vm_wait(int n) {
  return (n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8);
}

template <int ELEM>
__global__ void __launch_bounds__(64 * kStreamWaves)
block_matmul_f32b_stream(const uint8_t* __restrict__ a, const uint8_t* __restrict__ sa,
                         const float* __restrict__ b, float* __restrict__ c, int64_t M, int64_t N,
                         int64_t K, int accumulate, int tiles_n) {
  __shared__ __align__(1024) uint8_t lds[kStreamWaves * kWaveLds];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, q = lane >> 4;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int64_t m0 = (int64_t)tm * 16, n0 = (int64_t)tn * 16;
  const int64_t kb = K / 32, units = kb / 8;
  // Units are dealt to the waves in turn (wave w takes units w, w + 16, ...),
  // so that at small K the busy waves sit on different SIMDs.
  constexpr int kCodeBytes = ELEM == kE2M1 ? 16 : 32;  // per block and row
  constexpr int kCodeVecs = ELEM == kE2M1 ? 2 : 4;     // 16-byte loads per lane and unit

  const int64_t arow = min(m0 + r16, M - 1);
  const uint8_t* arow_codes = a + arow * kb * kCodeBytes;
  const uint8_t* arow_scales = sa + arow * kb;
  // Copy lane L of a 16-row run moves row L / 4, columns 4 (L % 4) .. + 3
  // (clamped to the last 4 columns; N % 4 == 0).
  const int64_t bcol = min(n0 + 4 * (lane & 3), N - 4);
  const uint32_t b_lane_off = (uint32_t)(((lane >> 2) * N + bcol) * 4);
  uint8_t* wl = lds + w * kWaveLds;
  const float* brow = reinterpret_cast<const float*>(wl + q * kRunBytes) + r16;

  v4f T = {0.f, 0.f, 0.f, 0.f}, G = {0.f, 0.f, 0.f, 0.f};
  int pending = 0;
  for (int64_t u = w; u < units; u += kStreamWaves) {
    const int64_t k0 = u * 256;
    // The unit's 256 rows of B as one buffer resource (256 N floats).
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(b + k0 * N), (short)0, (int)(256 * N * 4), 0x00020000);
    auto copy_quarter = [&](int qi) {
      uint8_t* st = wl + (qi & 1) * kStageBytes;
#pragma unroll
      for (int p = 0; p < 4; ++p)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rb, (__attribute__((address_space(3))) void*)(st + p * kRunBytes), 16, b_lane_off,
            (uint32_t)((64 * p + 16 * qi) * N * 4), 0, 0);
    };
    uint4 codes[kCodeVecs];
    const uint4* cp = reinterpret_cast<const uint4*>(arow_codes + (k0 / 32 + 2 * q) * kCodeBytes);
#pragma unroll
    for (int i = 0; i < kCodeVecs; ++i) codes[i] = cp[i];
    const uint32_t byte0 = arow_scales[k0 / 32 + 2 * q], byte1 = arow_scales[k0 / 32 + 2 * q + 1];
    // The previous unit's last LDS reads are complete (their MFMAs ran), but
    // keep the copies behind them explicitly.
    __builtin_amdgcn_s_waitcnt(kLgkm0);
    copy_quarter(0);
    copy_quarter(1);
#pragma unroll
    for (int qi = 0; qi < 4; ++qi) {
      // Loads still allowed in flight: the next quarter's 4 copies, if issued.
      if (qi < 3)
        __builtin_amdgcn_s_waitcnt(vm_wait(4));
      else
        __builtin_amdgcn_s_waitcnt(vm_wait(0));
      const float* bq = brow + (qi & 1) * (kStageBytes / 4);
      float bv[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) bv[t] = bq[t * 16];
      const int h = qi >> 1;
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const int ch = 2 * (qi & 1) + cc;  // chain within the block: its K 8ch .. 8ch + 7
        const uint32_t* cw = &codes[0].x;
        RawA r;
        r.byte = h ? byte1 : byte0;
        r.w0 = ELEM == kE2M1 ? cw[4 * h + ch] : cw[8 * h + 2 * ch];
        r.w1 = ELEM == kE2M1 ? 0u : cw[8 * h + 2 * ch + 1];
        float av[8];
        decode_a<ELEM>(av, r);
        v4f P = __builtin_amdgcn_mfma_f32_16x16x4f32(av[0], bv[8 * cc], v4f{0.f, 0.f, 0.f, 0.f},
                                                     0, 0, 0);
#pragma unroll
        for (int s = 1; s < 8; ++s)
          P = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s], bv[8 * cc + s], P, 0, 0, 0);
        G += P;
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);  // the quarter's 16 LDS reads first
      __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);  // then its 16 MFMAs
      if (qi < 2) {
        // This stage's reads are done before its next copy lands.
        __builtin_amdgcn_s_waitcnt(kLgkm0);
        copy_quarter(qi + 2);
      }
    }
    if (++pending == 2) {
      T += G;
      G = v4f{0.f, 0.f, 0.f, 0.f};
      pending = 0;
    }
  }
  T += G;

  // Partial sums of the 16 K ranges, added in wave order.
  __syncthreads();
  v4f* red = reinterpret_cast<v4f*>(lds);
  red[w * 64 + lane] = T;
  __syncthreads();
  if (w != 0) return;
  v4f sum = red[lane];
#pragma unroll
  for (int x = 1; x < kStreamWaves; ++x) sum += red[x * 64 + lane];
  const int64_t col = n0 + r16;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t row = m0 + 4 * q + r;
    if (row < M && col < N) {
      float v = sum[r];
      if (accumulate) v += c[row * N + col];
      c[row * N + col] = v;
    }
  }
}

template <int ELEM, int SPLIT, int TI, int TJ, int U>
hipError_t launch_shape(const uint8_t* a, const uint8_t* sa, const float* b, float* c, int64_t M,
                        int64_t N, int64_t K, int accumulate, hipStream_t stream) {
  constexpr int BM = (SPLIT == 1 ? 2 : 1) * TI * 16, BN = (SPLIT == 1 ? 2 : 1) * TJ * 16;
  const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  if (tiles_m * tiles_n > 0x7FFFFFFF || tiles_n > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((block_matmul_f32b_kernel<ELEM, SPLIT, TI, TJ, U>),
                     dim3((unsigned)(tiles_m * tiles_n)), dim3(f32b_threads<SPLIT>()), 0, stream,
                     a, sa, b, c,
                     M, N, K, accumulate, (int)tiles_n);
  return hipGetLastError();
}

template <int ELEM>
hipError_t launch_elem(const uint8_t* a, const uint8_t* sa, const float* b, float* c, int64_t M,
                       int64_t N, int64_t K, int accumulate, hipStream_t stream) {
  // 4x2 MFMA tiles per wave: measured fastest of 1x2, 2x2 (1.76 ms), 2x4, 4x2
  // (1.40 ms), 4x3, 4x4, 8x1 and 8x2 on the 4096^3 product.
  const int64_t big_tiles = ((M + 127) / 128) * ((N + 63) / 64);
  if (big_tiles >= 256)
    return launch_shape<ELEM, 1, 4, 2, 1>(a, sa, b, c, M, N, K, accumulate, stream);
  if (K % 256 == 0 && N % 4 == 0 && N <= (1 << 20) && reinterpret_cast<uintptr_t>(b) % 16 == 0) {
    const int64_t tiles_m = (M + 15) / 16, tiles_n = (N + 15) / 16;
    hipLaunchKernelGGL(block_matmul_f32b_stream<ELEM>, dim3((unsigned)(tiles_m * tiles_n)),
                       dim3(64 * kStreamWaves), 0, stream, a, sa, b, c, M, N, K, accumulate,
                       (int)tiles_n);
    return hipGetLastError();
  }
  // One block per load batch: measured fastest of 1, 2 and 4 (and of 4, 8
  // and 16 waves) on the 4096x4096 . 4096x16 decode shape.
  return launch_shape<ELEM, 16, 1, 1, 1>(a, sa, b, c, M, N, K, accumulate, stream);
}

}  // namespace

hipError_t launch_block_matmul_f32b(const void* a_codes, const uint8_t* a_scales, int a_elem,
                                    const float* b, float* c, int64_t M, int64_t N, int64_t K,
                                    int accumulate, hipStream_t stream) {
  const uint8_t* a = static_cast<const uint8_t*>(a_codes);
  if (a_elem == kE2M1)
    return launch_elem<kE2M1>(a, a_scales, b, c, M, N, K, accumulate, stream);
  return launch_elem<kE4M3>(a, a_scales, b, c, M, N, K, accumulate, stream);
}

}  // namespace mx
