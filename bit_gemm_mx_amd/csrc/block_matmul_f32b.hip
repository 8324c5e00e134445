// MX block matmul with an ordinary float32 B: C[M,N] (+)= A[M,K] . B[K,N],
// A block-scaled along K (codes + E8M0 scales), B row-major float32 [K, N].
// This is block_matmul as the dialect page "A Dialect Is a Set of
// Co-Designed Decisions" states its first version (section "The four ops":
// a block-scaled A of shape MxK, an ordinary f32 B of shape KxN, C += A.B;
// section "The accumulator operand": C is updated in place).
//
// Arithmetic: A's elements are decoded exactly (grid value x 2^(byte-127),
// by the hardware's scaled converts) and multiplied with B on the fp32 matrix
// cores (v_mfma_f32_16x16x4_f32), or, in the square-shape kernel further
// down, exactly on the bf16 ones with B split into three bf16 parts.  In the
// fp32 kernels each 32-element block of K is summed into a
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
// whole K each) when that gives at least one workgroup per CU -- on the bf16
// matrix cores when K % 128 == 0, N % 4 == 0 and B and A's scales are
// aligned (block_matmul_f32b_bf16), else on the fp32 ones; otherwise a
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

// ---------------------------------------------------------------------------
// Square-shape kernel on the bf16 matrix cores (many output tiles, K a
// multiple of 128, N a multiple of 4, B 16-byte and A's scales 4-byte
// aligned).  Same tiles as the 128x64 fp32 shape (4 waves of TI x 2 16x16
// tiles, whole K each), but every product a * b is computed exactly as
// a * hi + a * mid + a * lo, with b = hi + mid + lo split into three bf16
// values and a (a decoded MX value) itself a bf16 value, by three
// v_mfma_f32_16x16x32_bf16 per block of 32 K instead of eight
// v_mfma_f32_16x16x4_f32: the bf16 MFMA multiplies exactly and sums within
// 2^-24 of its largest term (probed).  Within each group of four blocks a
// tile's partial sum stays in the MFMA accumulator (at most 12 bf16 or 32
// fp32 MFMAs); groups are added in float32.  A block holding a value the
// split cannot carry exactly (E4M3 codes at scale bytes 0..2, B values whose
// last bits fall below the bf16 subnormals, infinities, NaNs, NaN scales)
// runs the float32 MFMAs instead, for the whole wave.
//
// Operands reach the waves through LDS: each wave copies, per block of 32 K,
// its 32 B rows x 32 columns (4 KiB), its 16 TI A rows' codes and their
// scale dwords (the block's group of four blocks) with buffer loads that
// write LDS directly, into a ring of stages of its own (no barriers: each
// wave waits on its own loads).  The 16-byte B loads replace eight dword
// loads per B column and lane group, which bound the register-loading kernel
// once its MFMA time dropped.  The B stage is laid out so that the 64 lanes
// reading one K step of one 16-column tile hit 64 different banks: row
// k = 8q + s (lane group q, step s) is stored as virtual row
// 2s + (q % 2) + 16 (q / 2), its 16-byte chunks XORed with 4 (q / 2).
// Measured on the 4096^3 MXFP4 x f32 product: 0.60 ms, against 1.40 ms for
// the float32 MFMA kernel and 1.02 ms for the bf16 split on operands loaded
// into registers.
// ---------------------------------------------------------------------------
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// Eight floats whose values are bf16 values (low 16 bits zero) as the eight
// bf16 of an MFMA operand: the high halves, element 0 in the low half of the
// first dword.
__device__ __forceinline__ v8bf pack_bf16(const float (&v)[8]) {
  uint32_t w[4];
#pragma unroll
  for (int p = 0; p < 4; ++p)
    w[p] = __builtin_amdgcn_perm(__float_as_uint(v[2 * p + 1]), __float_as_uint(v[2 * p]),
                                 0x07060302u);
  v8bf r;
  __builtin_memcpy(&r, w, 16);
  return r;
}

// decode_a's eight values as bf16, by the scaled converts to bf16: exact
// whenever the values are bf16 values (every E2M1 code at every scale byte,
// every E4M3 code at bytes 3..254; not for a NaN scale).
template <int ELEM>
__device__ __forceinline__ v8bf decode_a_bf16(const RawA& r) {
  const float sc = scale_value(r.byte);
  v2bf p0, p1, p2, p3;
  if (ELEM == kE2M1) {
    p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(r.w0, sc, 0);
    p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(r.w0, sc, 1);
    p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(r.w0, sc, 2);
    p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(r.w0, sc, 3);
  } else {
    p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.w0, sc, false);
    p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.w0, sc, true);
    p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.w1, sc, false);
    p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.w1, sc, true);
  }
  return v8bf{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

constexpr uint32_t kF32bOutOfRange = 0x80000000u;  // past every buffer resource here

// One stage (one block of 32 K) of a wave's ring: B 32 rows x 32 floats, A's
// 16 TI rows of codes, their scale dwords.
template <int ELEM, int TI>
struct F32bStage {
  static constexpr int kRows = 16 * TI;                  // A rows per wave
  static constexpr int kCodeBytes = ELEM == kE2M1 ? 16 : 32;  // per row and block
  static constexpr int kB = 4096;
  static constexpr int kA = kRows * kCodeBytes;
  static constexpr int kS = kRows * 4;
  static constexpr int kBytes = kB + kA + kS;
  static constexpr int kOps = 4 + kA / 1024 + kS / 256;  // load instructions per stage
  // Three stages per wave where two workgroups of 4 waves fit a CU, else two.
  static constexpr int kRing = 4 * 3 * kBytes <= 80 * 1024 ? 3 : 2;
};

// Exact three-way bf16 split of eight B values, and whether it holds (see
// above).  hi is b truncated to its top 8 significant bits and mid the next
// 8 (both subtractions remove a value's leading bits, so they are exact);
// lo, the rest, is a bf16 value when its low 16 bits are zero.
__device__ __forceinline__ void split_bf16(const float (&b)[8], v8bf& hi, v8bf& mid, v8bf& lo,
                                           bool& ok) {
  float h[8], m[8], l[8];
  uint32_t low = 0;
  bool finite = true;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    h[s] = __uint_as_float(__float_as_uint(b[s]) & 0xFFFF0000u);
    const float r = b[s] - h[s];
    m[s] = __uint_as_float(__float_as_uint(r) & 0xFFFF0000u);
    l[s] = r - m[s];
    low |= __float_as_uint(l[s]);
    finite = finite && !__builtin_amdgcn_class(b[s], 0x207);  // not NaN or +-Inf
  }
  ok = ok && finite && (low & 0xFFFFu) == 0;
  hi = pack_bf16(h);
  mid = pack_bf16(m);
  lo = pack_bf16(l);
}

template <int ELEM, int TI>
__global__ void __launch_bounds__(256)
block_matmul_f32b_bf16(const uint8_t* __restrict__ a, const uint8_t* __restrict__ sa,
                       const float* __restrict__ b, float* __restrict__ c, int64_t M, int64_t N,
                       int64_t K, int accumulate, int tiles_n) {
  using S = F32bStage<ELEM, TI>;
  constexpr int TJ = 2, kRing = S::kRing, kCodeBytes = S::kCodeBytes;
  __shared__ __align__(1024) uint8_t lds[4 * kRing * S::kBytes];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, q = lane >> 4;
  const int wm = w >> 1, wn = w & 1;
  // Tile order: each XCD (workgroups are dealt to the 8 XCDs in turn) takes
  // a contiguous range of tiles, walked in groups of 4 tile-rows, so that
  // the tiles running together on one XCD share B's columns and A's rows in
  // its L2 (measured 0.59 against 0.63 ms on the 4096^3 product; groups of
  // 2, 8, 16 and 32 rows 0.60-0.62).
  const int tiles_m = gridDim.x / tiles_n;
  const int nwg = tiles_m * tiles_n;
  int pid = blockIdx.x;
  if ((nwg & 7) == 0) pid = (pid & 7) * (nwg >> 3) + (pid >> 3);
  constexpr int kGroup = 4;
  const int in_group = kGroup * tiles_n;
  const int first_m = (pid / in_group) * kGroup;
  const int gsize = min(tiles_m - first_m, kGroup);
  const int tm = first_m + (pid % in_group) % gsize;
  const int tn = (pid % in_group) / gsize;
  const int64_t m0 = (int64_t)tm * (2 * S::kRows) + wm * S::kRows, n0 = (int64_t)tn * 64 + wn * 32;
  const int64_t kb = K / 32;
  const uint32_t row_bytes = (uint32_t)(kb * kCodeBytes);
  uint8_t* const ring = lds + w * kRing * S::kBytes;

  // A: this wave's 16 TI rows (rows past M read as zeros).
  const int64_t a_rows = M - m0 < S::kRows ? (M - m0 > 0 ? M - m0 : 0) : S::kRows;
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a + (M > m0 ? m0 : 0) * row_bytes), (short)0, (int)(a_rows * row_bytes),
      0x00020000);
  const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(sa + (M > m0 ? m0 : 0) * kb), (short)0, (int)(a_rows * kb), 0x00020000);
  // B stage lane offsets: instruction p, lane l writes virtual row 8p + l/8,
  // chunk position l % 8, i.e. B row k = 8 qq + ss, columns 4 cc .. 4 cc + 3.
  uint32_t b_off[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int vrow = 8 * p + (lane >> 3), cp = lane & 7;
    const int qq = 2 * (vrow >> 4) + (vrow & 1), ss = (vrow & 15) >> 1;
    const int cc = cp ^ (4 * (qq >> 1));
    b_off[p] = (uint32_t)(((8 * qq + ss) * N + 4 * cc) * 4);
  }
  // A stage: row-major, 16 or 32 code bytes per row, 1 KiB per load
  // instruction (64 or 32 rows); scale dwords: 64 rows per instruction.
  const uint32_t a_lane = ELEM == kE2M1 ? (uint32_t)lane * row_bytes
                                        : (uint32_t)(lane >> 1) * row_bytes + 16u * (lane & 1);
  constexpr int kRowsPerA = 1024 / kCodeBytes;
  const uint32_t s_lane = (uint32_t)lane * (uint32_t)kb;
  const int64_t b_cols = N - n0;  // columns of B from n0 on (B rows are N floats)

  auto issue = [&](int64_t j, int slot) {
    uint8_t* st = ring + slot * S::kBytes;
    // B rows 32 j .. 32 j + 31 from column n0 on; blocks past K read nothing.
    const int64_t rows = j < kb ? 32 : 0;
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(b + 32 * j * N + n0), (short)0,
        (int)(rows == 0 ? 0 : (31 * N + b_cols) * 4), 0x00020000);
#pragma unroll
    for (int p = 0; p < 4; ++p)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rb, (__attribute__((address_space(3))) void*)(st + 1024 * p), 16, b_off[p], 0, 0, 0);
#pragma unroll
    for (int h = 0; h < S::kA / 1024; ++h)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, (__attribute__((address_space(3))) void*)(st + S::kB + 1024 * h), 16,
          j < kb ? a_lane + (uint32_t)(h * kRowsPerA) * row_bytes + (uint32_t)(j * kCodeBytes)
                 : kF32bOutOfRange,
          0, 0, 0);
#pragma unroll
    for (int h = 0; h < S::kS / 256; ++h)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsa, (__attribute__((address_space(3))) void*)(st + S::kB + S::kA + 256 * h), 4,
          j < kb ? s_lane + (uint32_t)(64 * h) * (uint32_t)kb + (uint32_t)(4 * (j / 4))
                 : kF32bOutOfRange,
          0, 0, 0);
  };

  v4f T[TI][TJ], G[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int t = 0; t < TJ; ++t) T[i][t] = G[i][t] = v4f{0.f, 0.f, 0.f, 0.f};

  // LDS read offsets of this lane's B values: tile t, step s.
  const int vq = (q & 1) + 16 * (q >> 1), xq = 4 * (q >> 1);

#pragma unroll
  for (int p = 0; p < kRing - 1; ++p) issue(p, p);
  int slot = 0;
  // Blocks in groups of four (K % 128 == 0): within a group each tile's
  // partial sum G runs through the MFMAs' accumulator (at most 12 bf16 or
  // 32 fp32 MFMAs, each adding its products within 2^-24 of its largest
  // term), and the groups are added into T in float32.
  for (int64_t jg = 0; jg < kb; jg += 4) {
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const int64_t j = jg + j4;
      // Stage j + ring - 1 goes into the slot stage j - 1 used (its reads are done).
      __builtin_amdgcn_s_waitcnt(kLgkm0);
      issue(j + kRing - 1, slot == 0 ? kRing - 1 : slot - 1);
      __builtin_amdgcn_s_waitcnt(vm_wait((kRing - 1) * S::kOps));
      const uint8_t* st = ring + slot * S::kBytes;
      float bv[TJ][8];
#pragma unroll
      for (int t = 0; t < TJ; ++t)
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int cp = (4 * t + (r16 >> 2)) ^ xq;
          bv[t][s] =
              *reinterpret_cast<const float*>(st + 4 * ((2 * s + vq) * 32 + 4 * cp + (r16 & 3)));
        }
      RawA ra_[TI];
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const int row = 16 * i + r16;
        if (ELEM == kE2M1) {
          ra_[i].w0 = *reinterpret_cast<const uint32_t*>(st + S::kB + row * 16 + 4 * q);
          ra_[i].w1 = 0;
        } else {
          const uint2 v = *reinterpret_cast<const uint2*>(st + S::kB + row * 32 + 8 * q);
          ra_[i].w0 = v.x;
          ra_[i].w1 = v.y;
        }
        ra_[i].byte =
            (*reinterpret_cast<const uint32_t*>(st + S::kB + S::kA + 4 * row) >> (8 * j4)) & 0xFFu;
      }
      bool ok = true;
      v8bf bh[TJ], bm[TJ], bl[TJ];
#pragma unroll
      for (int t = 0; t < TJ; ++t) split_bf16(bv[t], bh[t], bm[t], bl[t], ok);
      // (zero codes decode to zero at any scale: rows past M read zero codes
      // and zero scale bytes)
#pragma unroll
      for (int i = 0; i < TI; ++i)
        ok = ok && ra_[i].byte != 0xFFu &&
             (ELEM == kE2M1 || ra_[i].byte >= 3u || (ra_[i].w0 | ra_[i].w1) == 0u);
      if (__builtin_amdgcn_ballot_w64(!ok) == 0) {
#pragma unroll
        for (int i = 0; i < TI; ++i) {
          const v8bf ab = decode_a_bf16<ELEM>(ra_[i]);
#pragma unroll
          for (int t = 0; t < TJ; ++t) {
            v4f P = j4 == 0 ? v4f{0.f, 0.f, 0.f, 0.f} : G[i][t];
            P = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ab, bh[t], P, 0, 0, 0);
            P = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ab, bm[t], P, 0, 0, 0);
            G[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ab, bl[t], P, 0, 0, 0);
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < TI; ++i) {
          float av[8];
          decode_a<ELEM>(av, ra_[i]);
#pragma unroll
          for (int t = 0; t < TJ; ++t) {
            v4f P = j4 == 0 ? v4f{0.f, 0.f, 0.f, 0.f} : G[i][t];
#pragma unroll
            for (int s = 0; s < 8; ++s)
              P = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s], bv[t][s], P, 0, 0, 0);
            G[i][t] = P;
          }
        }
      }
      slot = slot == kRing - 1 ? 0 : slot + 1;
    }
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int t = 0; t < TJ; ++t) T[i][t] += G[i][t];
  }
  // No load may still be writing this wave's LDS when it exits.
  __builtin_amdgcn_s_waitcnt(vm_wait(0));
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
  const int64_t code_row = ELEM == kE2M1 ? K / 2 : K;
  if (big_tiles >= 256 && K % 128 == 0 && N % 4 == 0 && 32 * N * 4 < (1ll << 31) &&
      128 * code_row < (1ll << 31) && reinterpret_cast<uintptr_t>(b) % 16 == 0 &&
      reinterpret_cast<uintptr_t>(sa) % 4 == 0) {
    // Four A tiles per wave (TI = 8, one wave per SIMD: 0.578 against
    // 0.595 ms on the 4096^3 product, and two stages for E4M3).
    constexpr int TI = 4;
    const int64_t tiles_m = (M + 32 * TI - 1) / (32 * TI), tiles_n = (N + 63) / 64;
    if (tiles_m * tiles_n > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL((block_matmul_f32b_bf16<ELEM, TI>), dim3((unsigned)(tiles_m * tiles_n)),
                       dim3(256), 0, stream, a, sa, b, c, M, N, K, accumulate, (int)tiles_n);
    return hipGetLastError();
  }
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
