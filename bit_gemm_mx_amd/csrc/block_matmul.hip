// MX block matmul: C[M,N] (+)= A[M,K] . B[K,N], A and B^T [N,K] block-scaled
// along K, on CDNA4's block-scaled MFMA (v_mfma_scale_f32_*_f8f6f4).
//
// Semantics: the dialect page "A Dialect Is a Set of Co-Designed Decisions",
// sections "The four ops" (block_matmul, C += A.B) and "The block axis" (the
// scale of A[m,k] is S[m, k/32], constant along each 32-run of the reduction,
// so it multiplies that run's partial sum).  The scaled MFMA takes that form:
// each lane hands the instruction part of a row's K range plus the E8M0 byte
// of one 32-element block, and the instruction applies the block scales.
//
// Operand layouts, established with one-hot probes on gfx950 (G = 16 for the
// 16x16x128 shape, 32 for 32x32x64; lane group g = l / G, row = l % G; KS =
// the instruction's K extent):
//   * FP4 operands fill the first 4 VGPRs: lane l holds the 32 K elements
//     [32g, 32g+32) of its row, element 2i in the low nibble of byte i -- the
//     packing of the codes in memory, so one 16-byte load fills them.
//   * FP8 operands fill 8 VGPRs: bytes 0..15 hold K [16g, 16g+16) and bytes
//     16..31 hold K [KS/2 + 16g, KS/2 + 16g + 16) of the row.
//   * The scale operand of lane l carries the E8M0 byte of block g (K [32g,
//     32g+32)) of its row, in the byte that op_sel selects, for either format.
//   * Output: 16x16x128 -> lane l holds C[4g + j][l % 16], j = 0..3;
//     32x32x64 -> C[8(j/4) + 4g + (j%4)][l % 32], j = 0..15.
// B^T rows use the same layout as A rows (B column n = B^T row n).  A 0xFF
// scale or an E4M3 NaN code makes the affected outputs NaN in hardware.
#include <atomic>
#include <type_traits>
#include <utility>

#include "codec_common.h"
#include "mx_internal.h"

namespace mx {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// MFMA format selectors.
constexpr int kFmtFp8 = 0;  // E4M3
constexpr int kFmtFp4 = 4;  // E2M1

template <int ELEM>
struct Operand {
  static constexpr int kFmt = ELEM == kE2M1 ? kFmtFp4 : kFmtFp8;
};

// Exact products for E4M3 x E2M1.  Measured on gfx950 (one-hot and random
// probes of v_mfma_scale_f32_32x32x64_f8f6f4): the instruction adds the
// products of each aligned group of 8 consecutive K in fixed point whose
// lowest bit is 2^(X - 13), X the largest exponent sum (element exponents
// plus block scales) in the group, truncating every product toward zero to
// that grid; the group sums then go into the fp32 accumulator.  An E4M3 x
// E2M1 product carries 4 + 2 significant bits, its lowest at 2^(x_a + x_b
// - 4), so it is exact whenever x_a + x_b >= X - 9.  E2M1 exponents span 2
// (values 0.5 .. 6), so a group whose E4M3 exponents span at most 7 sums
// exactly.  Splitting every E4M3 code on bit 6 of its magnitude (exponent
// field >= 8, i.e. |q| >= 2, or not) gives two operands whose exponents
// span [1, 8] and [-6, 0]: each group of either is exact, the two add up to
// the original codes (the other part holds a zero code), and the block
// products then differ from the oracle only by the fp32 rounding of the
// accumulation.  (E4M3 x E4M3 products span 14 exponents per operand and
// have no split of this kind into few parts; they keep one instruction.)
__device__ __forceinline__ int e4m3_high(int w) {
  const uint32_t m = (uint32_t)w & 0x40404040u;   // bit 6 of each code byte
  return (int)((uint32_t)w & ((m << 2) - (m >> 6)));  // 0xFF where that bit is set
}
__device__ __forceinline__ v8i e4m3_high(v8i v) {
  v8i r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = e4m3_high(v[i]);
  return r;
}

// Which operand of an (A, B) format pair is split (the E4M3 one of a mixed
// pair), or neither.
template <int AE, int BE>
struct Split {
  static constexpr bool kA = AE == kE4M3 && BE == kE2M1;
  static constexpr bool kB = AE == kE2M1 && BE == kE4M3;
};

// Load lane group g's share of one 128-wide K step (starting at element k0)
// of row `row` of a [rows, K] code matrix; zeros outside the matrix.
template <int ELEM>
__device__ __forceinline__ v8i load_operand(const uint8_t* codes, int64_t row, int64_t rows,
                                            int64_t k0, int g, int64_t K) {
  v8i r = {0, 0, 0, 0, 0, 0, 0, 0};
  if (row >= rows) return r;
  if (ELEM == kE2M1) {
    const int64_t k = k0 + 32 * g;
    if (k < K) {
      const int4 v = *reinterpret_cast<const int4*>(codes + (row * K + k) / 2);
      r[0] = v.x; r[1] = v.y; r[2] = v.z; r[3] = v.w;
    }
  } else {
    const int64_t klo = k0 + 16 * g, khi = k0 + 64 + 16 * g;
    if (klo < K) {
      const int4 v = *reinterpret_cast<const int4*>(codes + row * K + klo);
      r[0] = v.x; r[1] = v.y; r[2] = v.z; r[3] = v.w;
    }
    if (khi < K) {
      const int4 v = *reinterpret_cast<const int4*>(codes + row * K + khi);
      r[4] = v.x; r[5] = v.y; r[6] = v.z; r[7] = v.w;
    }
  }
  return r;
}

__device__ __forceinline__ int load_scale(const uint8_t* scales, int64_t row, int64_t rows,
                                          int64_t kb, int64_t kblocks) {
  return (row < rows && kb < kblocks) ? (int)scales[row * kblocks + kb] : 127;
}

// ---------------------------------------------------------------------------
// Skinny kernel, for few rows of A (token-by-token decode) and for the shapes
// the tiled kernel does not take.  Such a product streams B once and is bound
// by how fast B arrives, so the design goal is many loads in flight early,
// each touching as few cache lines as possible:
//   * a workgroup of 8 waves owns 16 columns of C and up to 64 rows (T tiles
//     of the 16x16x128 scaled MFMA); its waves split K into 8 contiguous
//     ranges, each wave issues the loads of U K steps at once and then runs
//     their MFMAs, and the 8 partial tiles are summed in LDS in a fixed order
//     (so results are reproducible bit for bit);
//   * loads use a "quad" layout -- lane 4r + q fetches 16-byte chunk q of
//     row r, so each group of four lanes reads one contiguous 64-byte piece
//     -- and a cross-lane permute (ds_bpermute) moves the chunks into the
//     MFMA layout (lane 16g + r holds chunk g of row r).  Loading in the MFMA
//     layout directly would have every four lanes touch four rows;
//   * scale bytes travel the same way, one dword (one K step's four blocks)
//     per lane when rows of scales are dword aligned.
// Each B^T row slice is loaded once and used for all T row tiles of A.
// ---------------------------------------------------------------------------
constexpr int kSkinnyWaves = 8;
constexpr int kSkinnyThreads = 64 * kSkinnyWaves;

// Lane-permute one dword: every lane receives `v` of lane `addr / 4`.
__device__ __forceinline__ int lane_fetch(int addr, int v) {
  return __builtin_amdgcn_ds_bpermute(addr, v);
}

template <int ELEM>
__device__ __forceinline__ v8i to_mfma_layout(v8i v, int addr) {
  v8i r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (ELEM == kE2M1 && i >= 4) ? 0 : lane_fetch(addr, v[i]);
  return r;
}

// Scale dword of K step s of row `row` (its four blocks), or 127s outside.
__device__ __forceinline__ int load_scale_dword(const uint8_t* scales, int64_t row, int64_t rows,
                                                int64_t s, int64_t kblocks) {
  return row < rows ? (int)*reinterpret_cast<const uint32_t*>(scales + row * kblocks + 4 * s)
                    : 0x7F7F7F7F;
}

template <int AE, int BE, int T>
__global__ void __launch_bounds__(kSkinnyThreads)
block_matmul_skinny(const uint8_t* __restrict__ a, const uint8_t* __restrict__ sa,
                    const uint8_t* __restrict__ b, const uint8_t* __restrict__ sb,
                    float* __restrict__ c, int64_t M, int64_t N, int64_t K, int accumulate,
                    int scale_dwords) {
  // K steps per load batch: fewer when many row tiles share the registers.
  constexpr int U = T >= 4 ? 2 : 4;
  __shared__ v4f red[kSkinnyWaves][T][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int qr = lane >> 2, q = lane & 3;            // load layout: row qr, chunk q
  const int to_mfma = 4 * (4 * (lane & 15) + (lane >> 4));  // source lane (x4) of my MFMA slot
  const int gshift = 8 * (lane >> 4);                // my block within a step's scale dword
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t kblocks = K / 32;
  const int64_t steps = (kblocks + 3) / 4;  // 128-element MFMA K steps
  const int64_t per_wave = (steps + kSkinnyWaves - 1) / kSkinnyWaves;
  const int64_t s_begin = wave * per_wave;
  const int64_t s_end = min(steps, s_begin + per_wave);
  const int64_t brow = n0 + qr;

  for (int64_t m0 = (int64_t)blockIdx.y * 16 * T; m0 < M; m0 += (int64_t)gridDim.y * 16 * T) {
    v4f acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int64_t s0 = s_begin; s0 < s_end; s0 += U) {
      // Scale loads first (in-order load counters: their permutes then only
      // wait for them), then the operand loads, then permutes and MFMAs.
      // Dword path (kblocks % 4 == 0, aligned): lane 4r + q holds the four
      // blocks of step s0 + q.  Byte path: lane 4r + q holds block q of each
      // step.
      int bsr[U], asr[U][T];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        bsr[u] = 0x7F7F7F7F;
#pragma unroll
        for (int t = 0; t < T; ++t) asr[u][t] = 0x7F7F7F7F;
      }
      if (scale_dwords) {
        if (q < U && s0 + q < s_end) {
          bsr[0] = load_scale_dword(sb, brow, N, s0 + q, kblocks);
#pragma unroll
          for (int t = 0; t < T; ++t)
            asr[0][t] = load_scale_dword(sa, m0 + 16 * t + qr, M, s0 + q, kblocks);
        }
      } else {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (s0 + u < s_end) {
            const int64_t kb = 4 * (s0 + u) + q;
            bsr[u] = load_scale(sb, brow, N, kb, kblocks);
#pragma unroll
            for (int t = 0; t < T; ++t) asr[u][t] = load_scale(sa, m0 + 16 * t + qr, M, kb, kblocks);
          }
        }
      }
      v8i bv[U], av[U][T];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        bv[u] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int t = 0; t < T; ++t) av[u][t] = bv[u];
        if (s0 + u < s_end) {  // wave-uniform
          bv[u] = load_operand<BE>(b, brow, N, 128 * (s0 + u), q, K);
#pragma unroll
          for (int t = 0; t < T; ++t)
            av[u][t] = load_operand<AE>(a, m0 + 16 * t + qr, M, 128 * (s0 + u), q, K);
        }
      }
      int bs[U], as[U][T];
      if (scale_dwords) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int from = 4 * (4 * (lane & 15) + u);
          bs[u] = lane_fetch(from, bsr[0]) >> gshift;
#pragma unroll
          for (int t = 0; t < T; ++t) as[u][t] = lane_fetch(from, asr[0][t]) >> gshift;
        }
      } else {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          bs[u] = lane_fetch(to_mfma, bsr[u]);
#pragma unroll
          for (int t = 0; t < T; ++t) as[u][t] = lane_fetch(to_mfma, asr[u][t]);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (s0 + u < s_end) {
          const v8i bm = to_mfma_layout<BE>(bv[u], to_mfma);
          const v8i bh = Split<AE, BE>::kB ? e4m3_high(bm) : bm;
#pragma unroll
          for (int t = 0; t < T; ++t) {
            const v8i am = to_mfma_layout<AE>(av[u][t], to_mfma);
            if constexpr (Split<AE, BE>::kA) {
              const v8i ah = e4m3_high(am);
              acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                  ah, bm, acc[t], Operand<AE>::kFmt, Operand<BE>::kFmt, 0, as[u][t], 0, bs[u]);
              acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                  am ^ ah, bm, acc[t], Operand<AE>::kFmt, Operand<BE>::kFmt, 0, as[u][t], 0, bs[u]);
            } else if constexpr (Split<AE, BE>::kB) {
              acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                  am, bh, acc[t], Operand<AE>::kFmt, Operand<BE>::kFmt, 0, as[u][t], 0, bs[u]);
              acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                  am, bm ^ bh, acc[t], Operand<AE>::kFmt, Operand<BE>::kFmt, 0, as[u][t], 0, bs[u]);
            } else {
              acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                  am, bm, acc[t], Operand<AE>::kFmt, Operand<BE>::kFmt, 0, as[u][t], 0, bs[u]);
            }
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < T; ++t) red[wave][t][lane] = acc[t];
    __syncthreads();
    // Output o = (tile, row in tile, column): consecutive threads write
    // consecutive columns.  Lane l of a tile holds C[4(l/16) + j][l % 16].
    for (int o = threadIdx.x; o < T * 256; o += kSkinnyThreads) {
      const int t = o >> 8, rr = (o >> 4) & 15, cc = o & 15;
      const int src = 16 * (rr >> 2) + cc, j = rr & 3;
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kSkinnyWaves; ++w) v += red[w][t][src][j];
      const int64_t row = m0 + 16 * t + rr, col = n0 + cc;
      if (row < M && col < N) {
        if (accumulate) v += c[row * N + col];
        c[row * N + col] = v;
      }
    }
    __syncthreads();  // red is rewritten by the next row panel
  }
}

// ---------------------------------------------------------------------------
// Tiled kernel: TM x TN output tile (256 x 256, or 128 x 256 for a last
// round of tiles) per workgroup of WM x WN waves, each wave (TM / WM) x
// (TN / WN) of C = (TM / WM / 32) x (TN / WN / 32) tiles of the 32x32x64
// scaled MFMA.
//
// K runs in stages of TK elements (TK / 64 MFMA K steps).  Code tiles are
// staged straight into LDS by buffer loads that write LDS, two or four stage
// buffers deep (as many as fit; an FP8 x FP8 stage of 128 K is 64 KiB).
// Scale bytes are staged the same way, 16 per row (512 K elements, a "scale
// chunk" of 512 / TK stages) in one load per row, double-buffered by chunk
// parity.  Every global load of the main loop thus writes LDS and is covered
// by the explicit waits before the barriers; operand and scale registers only
// wait on LDS reads.
// ---------------------------------------------------------------------------
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));


template <int ELEM, int TK, int WAVES = 4, int ROWS = 256>
struct Stage {
  static constexpr int kRowBytes = ELEM == kE2M1 ? TK / 2 : TK;     // 32 .. 128
  static constexpr int kChunks = kRowBytes / 16;                     // 16-B chunks per row
  static constexpr int kRowsPerLine = 256 / kRowBytes;               // rows per 256-B line
  static constexpr int kBytes = ROWS * kRowBytes;                    // one ROWS-row tile
  static constexpr int kInstr = kBytes / 1024 / WAVES;               // 1-KiB loads per wave
  static_assert(kInstr * 1024 * WAVES == kBytes, "whole 1-KiB loads per wave");
};

// LDS byte offset of 16-byte chunk c of row r of a staged tile.  Rows are
// packed into 256-byte lines (the width the LDS serves per clock: 64 banks of
// 4 bytes, 16 lanes of a 16-byte read) and the chunk index within the line is
// XOR-swizzled with the line index, so that the 16 lanes reading the same
// logical chunk of 16 consecutive rows (an MFMA operand read) address 16
// different 16-byte bank groups.
template <int ELEM, int TK>
__device__ __forceinline__ int lds_off(int r, int c) {
  using S = Stage<ELEM, TK>;
  const int line = r / S::kRowsPerLine;
  const int q = (r % S::kRowsPerLine) * S::kChunks + c;
  return line * 256 + ((q ^ (line % S::kChunks)) << 4);
}

// Buffer resource over `bytes` bytes at `base` (raw buffer: offsets are byte
// offsets; loads at offsets past `bytes` return zeros).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

constexpr uint32_t kOutOfRange = 0x80000000u;  // past every resource used here

// Stage one ROWS-row tile of codes straight into LDS with buffer loads that
// write LDS directly (each wave instruction fills 1 KiB = 4 lines: lane i
// writes bytes [16i, 16i+16) of it).  LDS position (line L, chunk p) must hold
// logical chunk q = p ^ (L % kChunks) of row L * kRowsPerLine + q / kChunks, so
// each lane fetches that chunk from global memory.  Lane i covers line
// 4j + i/16 of instruction j; L % kChunks depends on the lane and, for 8 chunks
// per row, on the parity of j, so two lane offsets are kept.
template <int ELEM, int TK, int WAVES, int ROWS = 256>
struct Stager {
  using S = Stage<ELEM, TK, WAVES, ROWS>;
  uint32_t lane_off[2];  // row-in-instruction * row_bytes + 16 * chunk (even / odd j)
  uint32_t chunk16[2];   // 16 * chunk
  uint32_t instr_step;   // bytes between consecutive instructions' first rows

  __device__ __forceinline__ Stager(uint32_t row_bytes, int lane) {
#pragma unroll
    for (int odd = 0; odd < 2; ++odd) {
      const int line = 4 * odd + (lane >> 4);  // line within an 8-line period
      const int q = (lane & 15) ^ (line % S::kChunks);
      const int r = (lane >> 4) * S::kRowsPerLine + q / S::kChunks;
      const int c = q % S::kChunks;
      chunk16[odd] = 16u * c;
      lane_off[odd] = (uint32_t)r * row_bytes + 16u * c;
    }
    instr_step = 4 * S::kRowsPerLine * row_bytes;
  }

  // Stage whose first K byte (within each row) is byte0.  `rsrc` starts at
  // the tile's first row and ends at the matrix's last row, so rows past the
  // matrix read as zeros; chunks past K are sent out of range (zeros too).
  __device__ __forceinline__ void load(uint8_t* lds_tile, __amdgpu_buffer_rsrc_t rsrc,
                                       uint32_t row_bytes, uint32_t byte0, int wave) const {
#pragma unroll
    for (int j = 0; j < S::kInstr; ++j) {
      const int ji = wave * S::kInstr + j;
      const int odd = ji & 1;
      const uint32_t off =
          byte0 + chunk16[odd] < row_bytes ? lane_off[odd] + ji * instr_step : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc, (__attribute__((address_space(3))) void*)(lds_tile + ji * 1024), 16, off, byte0,
          0, 0);
    }
  }
};

// MFMA operand of row r for K step h of a staged tile.
template <int ELEM, int TK>
__device__ __forceinline__ v8i read_operand(const uint8_t* lds, int r, int h, int g) {
  if (ELEM == kE4M3) {
    const v4i lo = *reinterpret_cast<const v4i*>(lds + lds_off<ELEM, TK>(r, 4 * h + g));
    const v4i hi = *reinterpret_cast<const v4i*>(lds + lds_off<ELEM, TK>(r, 4 * h + 2 + g));
    return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  } else {
    const v4i lo = *reinterpret_cast<const v4i*>(lds + lds_off<ELEM, TK>(r, 2 * h + g));
    return v8i{lo.x, lo.y, lo.z, lo.w, 0, 0, 0, 0};
  }
}

// s_waitcnt immediate (gfx9 encoding) that waits until at most n vector
// memory operations are outstanding, leaving the other counters alone.
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
constexpr int kLgkmZero = 0xC07F;  // s_waitcnt lgkmcnt(0), other counters untouched

// Scale staging.  Chunk mode (K a multiple of 512): one 16-byte slice per row
// (16 blocks = 512 K) per chunk of stages, in two chunk buffers by parity.
// Stage mode (K a multiple of 128, DW): one dword per row (the stage's 4
// blocks) with every stage, stored after the stage's code tiles in the same
// stage buffer.
template <int AE, int BE, int TK, int WM, int WN, bool DW, int TM, int TN>
struct Pipe {
  static constexpr int kTK = TK;
  static constexpr int kWaves = WM * WN;                 // WM along M, WN along N
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kWaveM = TM / WM;                 // rows of C per wave
  static constexpr int kMQ = kWaveM / 32;                // 32x32 MFMA tiles along M per wave
  static_assert(kMQ >= 1 && kMQ * 32 * WM == TM, "whole 32-row MFMA tiles per wave");
  static constexpr int kWaveN = TN / WN;                 // columns of C per wave
  static constexpr int kNQ = kWaveN / 32;                // 32x32 MFMA tiles along N per wave
  static_assert(kNQ >= 1 && kNQ * 32 * WN == TN, "whole 32-column MFMA tiles per wave");
  static constexpr int kSteps = kTK / 64;                // MFMA K steps per stage
  static_assert(!DW || kTK == 128, "stage-mode scales hold one dword (4 blocks) per row");
  static constexpr int kChunkStages = DW ? 1 : 512 / kTK;  // stages per scale chunk
  static constexpr int kScaleRowBytes = DW ? 4 : 16;     // scale bytes per row per chunk
  static constexpr int kScaleBytes = 2 * 256 * kScaleRowBytes;  // A and B^T rows of a chunk
  static constexpr int kAB = Stage<AE, kTK, 4, TM>::kBytes + Stage<BE, kTK, 4, TN>::kBytes;
  static constexpr int kBuf = kAB + (DW ? kScaleBytes : 0);    // one stage buffer
  // As many stage buffers (4 or 2) as fit in 160 KiB (with two scale chunks).
  static constexpr int kStages = 4 * kBuf + (DW ? 0 : 2 * kScaleBytes) <= 160 * 1024 ? 4 : 2;
  // Stages walked per loop iteration: whole scale chunks of both parities.
  static constexpr int kUnroll = 2 * kChunkStages > kStages ? 2 * kChunkStages : kStages;
  static_assert(kUnroll % kStages == 0, "buffer slots must repeat within the unrolled body");
  static constexpr int kDma =
      Stage<AE, kTK, kWaves, TM>::kInstr + Stage<BE, kTK, kWaves, TN>::kInstr;
  // Scale chunk: 512 rows (A then B^T), 64 rows per load.
  static constexpr int kScaleDma = 8 / kWaves;           // per wave and chunk
  // Loads a wave issues along with stage s: its code tiles, plus the scale
  // chunk that starts with it.
  static constexpr int ops(int s) { return kDma + (s % kChunkStages == 0 ? kScaleDma : 0); }
  // Outstanding loads allowed when stage s starts: those of stages
  // s+1 .. s+kStages-2 (issued earlier, kStages-1 stages ahead).
  static constexpr int pending(int s) {
    int n = 0;
    for (int d = 1; d <= kStages - 2; ++d) n += ops(s + d);
    return n;
  }
};

template <typename F, int... U>
__device__ __forceinline__ void unroll_seq(F&& f, std::integer_sequence<int, U...>) {
  (f(std::integral_constant<int, U>{}), ...);
}

template <int AE, int BE, int TK, int WM, int WN, bool DW, int TM, int TN>
__global__ void __launch_bounds__(64 * WM * WN)
block_matmul_tiled(const uint8_t* __restrict__ a, const uint8_t* __restrict__ sa,
                   const uint8_t* __restrict__ b, const uint8_t* __restrict__ sb,
                   float* __restrict__ c, int64_t M, int64_t N, int64_t K, int64_t ldc,
                   int accumulate, int tiles_m, int tiles_n) {
  using P = Pipe<AE, BE, TK, WM, WN, DW, TM, TN>;
  constexpr int kTK = P::kTK, kChunkStages = P::kChunkStages, kWaves = P::kWaves;
  constexpr int kA = Stage<AE, kTK, 4, TM>::kBytes, kAB = P::kAB, kStages = P::kStages;
  constexpr int kMQ = P::kMQ, kNQ = P::kNQ, kBuf = P::kBuf;
  constexpr int kScaleRowBytes = P::kScaleRowBytes, kScaleBytes = P::kScaleBytes;
  // One array per buffer, always indexed by a compile-time slot, so that the
  // compiler can tell the direct-to-LDS loads into one buffer from the reads
  // of another and keep the loads in flight.
  __shared__ __attribute__((aligned(1024))) uint8_t smem0[kBuf];
  __shared__ __attribute__((aligned(1024))) uint8_t smem1[kBuf];
  __shared__ __attribute__((aligned(1024))) uint8_t smem2[kStages > 2 ? kBuf : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t smem3[kStages > 3 ? kBuf : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t scales0[DW ? 16 : kScaleBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t scales1[DW ? 16 : kScaleBytes];

  // Tile order: the hardware deals workgroups round-robin to the 8 XCDs, so
  // give each XCD a contiguous range of tiles, walked in groups of up to 4
  // tile-rows so that concurrently running tiles share A rows and B columns
  // in that XCD's L2 (groups of 4 measured ~2% faster than 8 on the 8192^3
  // FP8 product and the prefill product, 2 about the same, 16 7% slower).
  const int nwg = tiles_m * tiles_n;
  int pid = blockIdx.x;
  if ((nwg & 7) == 0) pid = (pid & 7) * (nwg >> 3) + (pid >> 3);
  constexpr int kGroup = 4;
  const int in_group = kGroup * tiles_n;
  const int first_m = (pid / in_group) * kGroup;
  const int gsize = min(tiles_m - first_m, kGroup);
  const int tm = first_m + (pid % in_group) % gsize;
  const int tn = (pid % in_group) / gsize;
  const int64_t m0 = (int64_t)tm * TM, n0 = (int64_t)tn * TN;

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave / WN, wn = wave % WN, g = lane >> 5, lr = lane & 31;
  const uint32_t Ku = (uint32_t)K;
  const uint32_t a_row_bytes = AE == kE2M1 ? Ku / 2 : Ku;
  const uint32_t b_row_bytes = BE == kE2M1 ? Ku / 2 : Ku;
  const Stager<AE, kTK, kWaves, TM> stage_a(a_row_bytes, lane);
  const Stager<BE, kTK, kWaves, TN> stage_b(b_row_bytes, lane);
  const uint32_t kblocks = Ku / 32;
  const int64_t rows_a = min(M - m0, (int64_t)TM), rows_b = min(N - n0, (int64_t)TN);
  // (a 256-row slab of either operand is below 2^31 bytes: checked at launch)
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a + m0 * a_row_bytes, rows_a * a_row_bytes);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(b + n0 * b_row_bytes, rows_b * b_row_bytes);
  const __amdgpu_buffer_rsrc_t rsa = make_rsrc(sa + m0 * kblocks, rows_a * kblocks);
  const __amdgpu_buffer_rsrc_t rsb = make_rsrc(sb + n0 * kblocks, rows_b * kblocks);
  // This lane's first A / B^T tile row.
  const int ar = wm * P::kWaveM + lr, br = wn * P::kWaveN + lr;

  v16f acc[kMQ][kNQ];
#pragma unroll
  for (int i = 0; i < kMQ; ++i)
#pragma unroll
    for (int j = 0; j < kNQ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  auto slot = [&](int buf) -> uint8_t* {
    return buf == 0 ? smem0 : buf == 1 ? smem1 : buf == 2 ? smem2 : smem3;
  };
  // Issue stage st into buffer (st % kStages); the first stage of a scale
  // chunk also fetches the chunk's scales into the set of the chunk's parity:
  // the 512 rows of the chunk (A's 256, then B^T's) as 16-byte row slices
  // (blocks [16 * chunk, 16 * chunk + 16)), 64 rows per load, rows in order.
  auto issue = [&](int st, int buf, int par) {
    uint8_t* dst = slot(buf);
    stage_a.load(dst, ra, a_row_bytes, (uint32_t)st * Stage<AE, kTK>::kRowBytes, wave);
    stage_b.load(dst + kA, rb, b_row_bytes, (uint32_t)st * Stage<BE, kTK>::kRowBytes, wave);
    if (st % kChunkStages == 0) {
      const uint32_t kb = (uint32_t)(st / kChunkStages) * kScaleRowBytes;
      uint8_t* sdst = DW ? dst + kAB : (par ? scales1 : scales0);
#pragma unroll
      for (int j = 0; j < P::kScaleDma; ++j) {
        const int part = wave * P::kScaleDma + j;  // 64-row part of the 512 rows
        const uint32_t off = kb < kblocks ? (uint32_t)(64 * (part & 3) + lane) * kblocks
                                          : kOutOfRange;
        auto* d = (__attribute__((address_space(3))) void*)(sdst + part * 64 * kScaleRowBytes);
        // Each size is a literal: a size that depends on a template parameter
        // is checked again when the host pass instantiates the kernel, which
        // rejects 16 (a gfx950-only size) and silently drops the launch stub.
        if constexpr (DW)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(part < 4 ? rsa : rsb, d, 4, off, kb, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(part < 4 ? rsa : rsb, d, 16, off, kb, 0, 0);
      }
    }
  };

  // The stage count is padded to whole loop iterations (kUnroll stages, 1024
  // K elements); stages past K load out of range (zero codes, zero scale
  // bytes) and add nothing.  Prologue: stages 0 .. kStages-2 in flight.
  const int iters = (int)((Ku + P::kUnroll * kTK - 1) / (P::kUnroll * kTK));
#pragma unroll
  for (int u = 0; u < kStages - 1; ++u) issue(u, u, 0);

  int it = 0;
  // Chunk-mode scales: each row's 16 bytes are read with one 16-byte LDS read
  // at the chunk's first stage and kept in registers for its other stages.
  // Dword reads per stage (16-byte row stride across 32 lanes) take 2-way
  // bank conflicts: the only bank conflicts of the kernel (SQ_LDS_BANK_CONFLICT
  // 1.9e7 -> 0 on the 8192^3 FP8 product).  Measured: E4M3 x E2M1 prefill
  // 373 -> 363 us; the FP8 x FP8 product 438 -> 442 us, so it keeps the
  // dword reads.
  // (Not for an E4M3 B: FP8 x FP8 measured faster with the dword reads, and
  // E2M1 x E4M3 needs the registers for its split B operand.)
  constexpr bool kScaleRegs = !DW && BE == kE2M1;
  v4i sa4[kMQ], sb4[kNQ];
  auto stage = [&](auto U) {
    constexpr int u = decltype(U)::value;
    constexpr int buf = u % kStages, par = u / kChunkStages % 2, sub = u % kChunkStages;
    constexpr int nu = u + kStages - 1;  // stage issued now, relative to the iteration
    const int st = it * P::kUnroll + u;
    // Wait for this stage's loads (later stages stay in flight), then make
    // them visible to every wave.  A bare s_barrier: a fenced __syncthreads
    // would also drain the later stages' loads.  The barrier also certifies
    // that every wave has consumed (in its MFMAs) its reads of the buffer the
    // issue below overwrites.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(P::pending(u)));
    __builtin_amdgcn_s_barrier();
    issue(st + kStages - 1, nu % kStages, nu / kChunkStages % 2);

    const uint8_t* la = slot(buf);
    const uint8_t* lb = la + kA;
    const uint8_t* sc = DW ? la + kAB : (par ? scales1 : scales0);
    // The stage covers blocks [blk0, blk0 + kTK/32) of the chunk.  Read the
    // scale dword holding them, shifted so that byte sel0 + 2h holds this
    // lane's block of K step h (lane group g takes block g of each step).
    constexpr int blk0 = sub * (kTK / 32), sel0 = blk0 % 4;
    int sas[kMQ], sbs[kNQ];
    if constexpr (!kScaleRegs) {
#pragma unroll
      for (int i = 0; i < kMQ; ++i)
        sas[i] = (int)(*reinterpret_cast<const uint32_t*>(sc + (ar + 32 * i) * kScaleRowBytes +
                                                          (blk0 & ~3)) >> (8 * g));
#pragma unroll
      for (int q = 0; q < kNQ; ++q)
        sbs[q] = (int)(*reinterpret_cast<const uint32_t*>(sc + kScaleBytes / 2 +
                                                          (br + 32 * q) * kScaleRowBytes +
                                                          (blk0 & ~3)) >> (8 * g));
    } else {
      if constexpr (sub == 0) {
#pragma unroll
        for (int i = 0; i < kMQ; ++i)
          sa4[i] = *reinterpret_cast<const v4i*>(sc + (ar + 32 * i) * kScaleRowBytes);
#pragma unroll
        for (int q = 0; q < kNQ; ++q)
          sb4[q] = *reinterpret_cast<const v4i*>(sc + kScaleBytes / 2 +
                                                 (br + 32 * q) * kScaleRowBytes);
      }
#pragma unroll
      for (int i = 0; i < kMQ; ++i) sas[i] = (int)((uint32_t)sa4[i][blk0 / 4] >> (8 * g));
#pragma unroll
      for (int q = 0; q < kNQ; ++q) sbs[q] = (int)((uint32_t)sb4[q][blk0 / 4] >> (8 * g));
    }
    auto kstep = [&](auto H) {
      constexpr int h = decltype(H)::value;
      v8i af[kMQ], bf[kNQ];
#pragma unroll
      for (int i = 0; i < kMQ; ++i) af[i] = read_operand<AE, kTK>(la, ar + 32 * i, h, g);
#pragma unroll
      for (int q = 0; q < kNQ; ++q) bf[q] = read_operand<BE, kTK>(lb, br + 32 * q, h, g);
      constexpr int sel = sel0 + 2 * h;
      constexpr int fa = Operand<AE>::kFmt, fb = Operand<BE>::kFmt;
      if constexpr (Split<AE, BE>::kA) {
#pragma unroll
        for (int i = 0; i < kMQ; ++i) {
          const v8i ah = e4m3_high(af[i]), al = af[i] ^ ah;
#pragma unroll
          for (int q = 0; q < kNQ; ++q) {
            acc[i][q] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                ah, bf[q], acc[i][q], fa, fb, sel, sas[i], sel, sbs[q]);
            acc[i][q] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                al, bf[q], acc[i][q], fa, fb, sel, sas[i], sel, sbs[q]);
          }
        }
      } else if constexpr (Split<AE, BE>::kB) {
#pragma unroll
        for (int q = 0; q < kNQ; ++q) {
          const v8i bh = e4m3_high(bf[q]), bl = bf[q] ^ bh;
#pragma unroll
          for (int i = 0; i < kMQ; ++i) {
            acc[i][q] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                af[i], bh, acc[i][q], fa, fb, sel, sas[i], sel, sbs[q]);
            acc[i][q] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                af[i], bl, acc[i][q], fa, fb, sel, sas[i], sel, sbs[q]);
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < kMQ; ++i)
#pragma unroll
          for (int q = 0; q < kNQ; ++q)
            acc[i][q] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                af[i], bf[q], acc[i][q], fa, fb, sel, sas[i], sel, sbs[q]);
      }
    };
    kstep(std::integral_constant<int, 0>{});
    if constexpr (P::kSteps > 1) kstep(std::integral_constant<int, 1>{});
    // Instruction order for the scheduler: the operand and scale reads of the
    // first K step, then one MFMA, one global load and one LDS read at a
    // time, so that the loads of the next stage drain through the memory
    // pipeline while the MFMAs run instead of stalling the wave in a burst.
    constexpr int kMfma = kMQ * kNQ * P::kSteps * (Split<AE, BE>::kA || Split<AE, BE>::kB ? 2 : 1);
    constexpr int kVmem = P::kDma + (nu % kChunkStages == 0 ? P::kScaleDma : 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);  // LDS reads
#pragma unroll
    for (int k = 0; k < kMfma; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);              // MFMA
      if (k < kVmem) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global load
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);              // LDS read
    }
  };
  for (; it < iters; ++it) unroll_seq(stage, std::make_integer_sequence<int, P::kUnroll>{});
  // No load may still be writing this workgroup's LDS when it exits.
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  // Epilogue: lane holds C[8(e/4) + 4g + (e%4)][lr] of each 32x32 tile, so
  // each store instruction writes two whole 128-byte row segments.  The
  // stores are non-temporal: C is written once and, stored through the
  // caches, would evict the operands that later tiles still read from the
  // Infinity Cache (measured 4% faster on the 8192^3 FP8 product).
#pragma unroll
  for (int i = 0; i < kMQ; ++i)
#pragma unroll
    for (int q = 0; q < kNQ; ++q) {
      const int64_t col = n0 + wn * P::kWaveN + 32 * q + lr;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = m0 + wm * P::kWaveM + 32 * i + 8 * (e >> 2) + 4 * g + (e & 3);
        if (row < M && col < N) {
          float v = acc[i][q][e];
          if (accumulate) v += c[row * ldc + col];
          __builtin_nontemporal_store(v, c + row * ldc + col);
        }
      }
    }
}

// Launch configuration: 128-element K stages, 8 waves.  Two waves per SIMD
// let one wave's MFMAs run while the other waits on LDS reads, its loads or
// the barrier.  Wave tiles are 128 x 64 of C (2 x 4 waves), or 64 x 128
// (4 x 2) when A's E4M3 codes are split: each wave then splits two A tiles
// per K step instead of four (the split is VALU work), and its LDS reads
// (two 32-byte A operands and four 16-byte E2M1 ones per lane) are 20%
// fewer.  The 128 x 256 tiles of a last round use 4 waves of the same wave
// tile; their stage (half of A's rows) is small enough for four stage
// buffers where a whole tile's E4M3 x E2M1 stage fits two.
constexpr int kTiledTK = 128;
constexpr int kTailTM = 128, kTailTN = 256;

template <int AE, int BE>
struct WaveGrid {
  static constexpr int kWM = Split<AE, BE>::kA ? 4 : 2;  // whole 256 x 256 tiles
  static constexpr int kWN = 8 / kWM;
  static constexpr int kTailWM = kWM / 2, kTailWN = kWN;  // 128 x 256 tiles
};

template <int AE, int BE, bool DW, int TM, int TN, int WM, int WN>
hipError_t launch_tiled(const uint8_t* a, const uint8_t* sa, const uint8_t* b, const uint8_t* sb,
                        float* c, int64_t M, int64_t N, int64_t K, int64_t ldc, int accumulate,
                        hipStream_t stream) {
  constexpr int TK = kTiledTK;
  const int64_t tiles_m = (M + TM - 1) / TM, tiles_n = (N + TN - 1) / TN;
  hipLaunchKernelGGL((block_matmul_tiled<AE, BE, TK, WM, WN, DW, TM, TN>),
                     dim3((unsigned)(tiles_m * tiles_n)),
                     dim3(Pipe<AE, BE, TK, WM, WN, DW, TM, TN>::kThreads), 0, stream, a, sa, b, sb,
                     c, M, N, K, ldc, accumulate, (int)tiles_m, (int)tiles_n);
  return hipGetLastError();
}

// Compute units of the current device (cached per device).
int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// One workgroup per compute unit at a time, so 256x256 tiles run in rounds
// of one tile per CU.  When the last round is at most half full (the
// 2048 x 28672 prefill product: 896 tiles = 3.5 rounds of 256 CUs), the tile
// columns holding it are computed by a second launch of 128x256 tiles, which
// fills the CUs in one round of half-size tiles; the rest of C is one launch
// of whole rounds.  The two launches write disjoint columns of C, and every
// output element sums the same MFMAs in the same K order as in one launch.
template <int AE, int BE, bool DW>
hipError_t launch_tiled_split(const uint8_t* a, const uint8_t* sa, const uint8_t* b,
                              const uint8_t* sb, float* c, int64_t M, int64_t N, int64_t K,
                              int accumulate, hipStream_t stream) {
  using G = WaveGrid<AE, BE>;
  const int64_t tiles_m = (M + 255) / 256, tiles_n = (N + 255) / 256;
  const int64_t tiles = tiles_m * tiles_n, cus = cu_count();
  const int64_t rem = tiles % cus;
  const int64_t tail_cols = (rem + tiles_m - 1) / tiles_m;  // tile columns of the last round
  const int64_t tail_wgs = (M + kTailTM - 1) / kTailTM * (tail_cols * 256 / kTailTN);
  if (tiles > cus && rem != 0 && tail_cols < tiles_n && tail_wgs <= cus) {
    const int64_t n1 = (tiles_n - tail_cols) * 256;
    const int64_t b_row_bytes = BE == kE2M1 ? K / 2 : K;
    const hipError_t e = launch_tiled<AE, BE, DW, 256, 256, G::kWM, G::kWN>(
        a, sa, b, sb, c, M, n1, K, N, accumulate, stream);
    if (e != hipSuccess) return e;
    return launch_tiled<AE, BE, DW, kTailTM, kTailTN, G::kTailWM, G::kTailWN>(
        a, sa, b + n1 * b_row_bytes, sb + n1 * (K / 32), c + n1, M, N - n1, K, N, accumulate,
        stream);
  }
  return launch_tiled<AE, BE, DW, 256, 256, G::kWM, G::kWN>(a, sa, b, sb, c, M, N, K, N,
                                                            accumulate, stream);
}

// ---------------------------------------------------------------------------
// Staged skinny kernel, for up to 32 rows of A (token-by-token decode) with K
// a multiple of 128.  The work split is the skinny kernel's (8 waves per 16
// columns of C, a contiguous range of K steps per wave, the 8 partial tiles
// summed in LDS in wave order), but the operands reach the MFMAs through LDS
// instead of register permutes:
//   * each wave stages a batch of U K steps (4, or 2 where two row tiles of
//     E4M3 codes would not fit the LDS) of its 16 B^T rows and 16 T A rows,
//     and their scale dwords, with buffer loads that write LDS directly.  One
//     16-byte load instruction fills 1 KiB, consecutive lanes reading a row's
//     whole span (128 to 512 contiguous bytes), so a batch touches the fewest
//     cache lines a row-major read can;
//   * after its own loads have landed (vmcnt; the region is the wave's own,
//     so no barrier), the wave reads each 32-element block of an MFMA
//     operand with one 16-byte LDS read, where the register path needs four
//     dword permutes for the same 16 bytes;
//   * 16-byte chunk c of row r of a staged span sits at chunk position
//     c ^ (r % 16) of that row (128-byte spans pair rows into 256-byte
//     lines), so the 16 lanes that read one block of 16 rows address 16
//     different bank groups;
//   * rows past the matrix read as zeros (the buffer range), their outputs
//     are not stored; K steps of a batch past the wave's range are multiplied
//     as zero codes (see the MFMA loop).
// ---------------------------------------------------------------------------
template <int AE, int BE, int T>
struct StagedSkinny {
  static constexpr int kStepA = AE == kE2M1 ? 64 : 128;  // bytes per row and 128-K step
  static constexpr int kStepB = BE == kE2M1 ? 64 : 128;
  // Per wave: B^T codes, A codes, then 16-byte scale rows of B^T and A.
  static constexpr int wave_bytes(int u) {
    return 16 * u * (T * kStepA + kStepB) + 256 * (1 + T);
  }
  static constexpr int kRed = kSkinnyWaves * T * 64 * 16;
  static constexpr int kU = kSkinnyWaves * wave_bytes(4) + kRed <= 160 * 1024 ? 4 : 2;
  static constexpr int kSpanA = kU * kStepA, kSpanB = kU * kStepB;  // 128 .. 512 bytes
  static constexpr int kCodesA = 16 * T * kSpanA, kCodesB = 16 * kSpanB;
  static constexpr int kWaveBytes = wave_bytes(kU);
  static_assert(kCodesA % 1024 == 0 && kCodesB % 1024 == 0, "whole 1-KiB load instructions");
};

// LDS offset of 16-byte chunk c of row r in a staged span of SPAN bytes per row.
template <int SPAN>
__device__ __forceinline__ int span_off(int r, int c) {
  if constexpr (SPAN >= 256) {
    return r * SPAN + ((c ^ (r & 15)) << 4);
  } else {
    static_assert(SPAN == 128, "spans of 128, 256 or 512 bytes");
    return (r >> 1) * 256 + (((((r & 1) << 3) | c) ^ ((r >> 1) & 7)) << 4);
  }
}

// Stage ROWS rows x SPAN bytes (from byte byte0 of each row) at `lds`: the
// lane that writes LDS offset o fetches the chunk span_off maps to o.
template <int SPAN, int ROWS, int AUX>
__device__ __forceinline__ void stage_span(uint8_t* lds, __amdgpu_buffer_rsrc_t rsrc,
                                           uint32_t row_bytes, uint32_t byte0, int lane) {
#pragma unroll
  for (int j = 0; j < ROWS * SPAN / 1024; ++j) {
    const int o = 1024 * j + 16 * lane;
    int r, c;
    if constexpr (SPAN >= 256) {
      r = o / SPAN;
      c = ((o % SPAN) >> 4) ^ (r & 15);
    } else {
      const int line = o >> 8, q = ((o & 255) >> 4) ^ (line & 7);
      r = 2 * line + (q >> 3);
      c = q & 7;
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc, (__attribute__((address_space(3))) void*)(lds + 1024 * j), 16,
        (uint32_t)r * row_bytes + byte0 + 16u * c, 0, 0, AUX);
  }
}

// MFMA operand (row r, K step u, lane group g) from a staged span.
template <int ELEM, int SPAN>
__device__ __forceinline__ v8i read_span(const uint8_t* lds, int r, int u, int g) {
  if constexpr (ELEM == kE4M3) {
    const v4i lo = *reinterpret_cast<const v4i*>(lds + span_off<SPAN>(r, 8 * u + g));
    const v4i hi = *reinterpret_cast<const v4i*>(lds + span_off<SPAN>(r, 8 * u + 4 + g));
    return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  } else {
    const v4i lo = *reinterpret_cast<const v4i*>(lds + span_off<SPAN>(r, 4 * u + g));
    return v8i{lo.x, lo.y, lo.z, lo.w, 0, 0, 0, 0};
  }
}

template <int AE, int BE, int T>
__global__ void __launch_bounds__(kSkinnyThreads)
block_matmul_skinny_staged(const uint8_t* __restrict__ a, const uint8_t* __restrict__ sa,
                           const uint8_t* __restrict__ b, const uint8_t* __restrict__ sb,
                           float* __restrict__ c, int64_t M, int64_t N, int64_t K,
                           int accumulate) {
  using S = StagedSkinny<AE, BE, T>;
  constexpr int U = S::kU;
  __shared__ __align__(1024) uint8_t lds[kSkinnyWaves * S::kWaveBytes];
  __shared__ v4f red[kSkinnyWaves][T][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t kblocks = K / 32, steps = K / 128;
  const int64_t per_wave = (steps + kSkinnyWaves - 1) / kSkinnyWaves;
  const int64_t s_begin = wave * per_wave;
  const int64_t s_end = min(steps, s_begin + per_wave);
  const uint32_t rb_a = (uint32_t)(K / 128 * S::kStepA), rb_b = (uint32_t)(K / 128 * S::kStepB);
  const int64_t rows_b = min((int64_t)16, N - n0), rows_a = min((int64_t)(16 * T), M);
  const __amdgpu_buffer_rsrc_t code_b = make_rsrc(b + n0 * rb_b, rows_b * rb_b);
  const __amdgpu_buffer_rsrc_t code_a = make_rsrc(a, rows_a * rb_a);
  const __amdgpu_buffer_rsrc_t scale_b = make_rsrc(sb + n0 * kblocks, rows_b * kblocks);
  const __amdgpu_buffer_rsrc_t scale_a = make_rsrc(sa, rows_a * kblocks);
  uint8_t* const lds_b = lds + wave * S::kWaveBytes;
  uint8_t* const lds_a = lds_b + S::kCodesB;
  uint8_t* const lds_sb = lds_a + S::kCodesA;
  uint8_t* const lds_sa = lds_sb + 256;
  // Scale load lane l: row l / 4 (of each 16-row group), step l % 4 of the batch.
  const int srow = lane >> 2, sstep = lane & 3;

  v4f acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int64_t s0 = s_begin; s0 < s_end; s0 += U) {
    const int n_steps = (int)min((int64_t)U, s_end - s0);  // wave-uniform
    stage_span<S::kSpanB, 16, 2>(lds_b, code_b, rb_b, (uint32_t)(s0 * S::kStepB), lane);
    stage_span<S::kSpanA, 16 * T, 0>(lds_a, code_a, rb_a, (uint32_t)(s0 * S::kStepA), lane);
    const uint32_t soff = (uint32_t)(4 * (s0 + sstep));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        scale_b, (__attribute__((address_space(3))) void*)lds_sb, 4,
        sstep < U ? (uint32_t)(srow * kblocks) + soff : kOutOfRange, 0, 0, 0);
#pragma unroll
    for (int t = 0; t < T; ++t)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          scale_a, (__attribute__((address_space(3))) void*)(lds_sa + 256 * t), 4,
          sstep < U ? (uint32_t)((16 * t + srow) * kblocks) + soff : kOutOfRange, 0, 0, 0);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    // All of the batch's LDS reads first (one round trip), then the MFMAs.
    // A step past the wave's range multiplies zero codes by zero codes at
    // scale 1 (its staged bytes belong to other steps or rows, NaN codes
    // included), adding +0 to accumulators that never hold -0, so the MFMA
    // sequence has no branch for the reads to sink behind.
    const v4i bsd = *reinterpret_cast<const v4i*>(lds_sb + 16 * r16);
    v4i asd[T];
#pragma unroll
    for (int t = 0; t < T; ++t)
      asd[t] = *reinterpret_cast<const v4i*>(lds_sa + 16 * (16 * t + r16));
    v8i bm[U], am[U][T];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      bm[u] = read_span<BE, S::kSpanB>(lds_b, r16, u, g);
#pragma unroll
      for (int t = 0; t < T; ++t) am[u][t] = read_span<AE, S::kSpanA>(lds_a, 16 * t + r16, u, g);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool live = u < n_steps;
      const int bs = live ? bsd[u] >> (8 * g) : 127;
      const v8i b_op = live ? bm[u] : v8i{0, 0, 0, 0, 0, 0, 0, 0};
      const v8i bh = Split<AE, BE>::kB ? e4m3_high(b_op) : b_op;
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const int as = live ? asd[t][u] >> (8 * g) : 127;
        const v8i a_op = live ? am[u][t] : v8i{0, 0, 0, 0, 0, 0, 0, 0};
        if constexpr (Split<AE, BE>::kA) {
          const v8i ah = e4m3_high(a_op);
          acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              ah, b_op, acc[t], Operand<AE>::kFmt, Operand<BE>::kFmt, 0, as, 0, bs);
          acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              a_op ^ ah, b_op, acc[t], Operand<AE>::kFmt, Operand<BE>::kFmt, 0, as, 0, bs);
        } else if constexpr (Split<AE, BE>::kB) {
          acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              a_op, bh, acc[t], Operand<AE>::kFmt, Operand<BE>::kFmt, 0, as, 0, bs);
          acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              a_op, b_op ^ bh, acc[t], Operand<AE>::kFmt, Operand<BE>::kFmt, 0, as, 0, bs);
        } else {
          acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              a_op, b_op, acc[t], Operand<AE>::kFmt, Operand<BE>::kFmt, 0, as, 0, bs);
        }
      }
    }
    // The next batch's loads overwrite this wave's LDS region: its reads are done.
    __builtin_amdgcn_s_waitcnt(kLgkmZero);
  }
#pragma unroll
  for (int t = 0; t < T; ++t) red[wave][t][lane] = acc[t];
  __syncthreads();
  for (int o = threadIdx.x; o < T * 256; o += kSkinnyThreads) {
    const int t = o >> 8, rr = (o >> 4) & 15, cc = o & 15;
    const int src = 16 * (rr >> 2) + cc, j = rr & 3;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kSkinnyWaves; ++w) v += red[w][t][src][j];
    const int64_t row = 16 * t + rr, col = n0 + cc;
    if (row < M && col < N) {
      if (accumulate) v += c[row * N + col];
      c[row * N + col] = v;
    }
  }
}

template <int AE, int BE>
hipError_t launch_skinny(const uint8_t* a, const uint8_t* sa, const uint8_t* b,
                         const uint8_t* sb, float* c, int64_t M, int64_t N, int64_t K,
                         int accumulate, hipStream_t stream) {
  const int64_t gx = (N + 15) / 16;
  if (gx > 0x7FFFFFFF) return hipErrorInvalidValue;
  const int t = M <= 16 ? 1 : M <= 32 ? 2 : 4;
  const int64_t panels = (M + 16 * t - 1) / (16 * t);
  const dim3 grid((unsigned)gx, (unsigned)(panels < 65535 ? panels : 65535));
  // Scale rows can be read a dword (one K step) at a time when every row
  // starts on a dword boundary and holds whole steps.
  const int dw = (K % 128 == 0) && ((reinterpret_cast<uintptr_t>(sa) & 3) == 0) &&
                 ((reinterpret_cast<uintptr_t>(sb) & 3) == 0);
  // The staged kernel addresses 32 rows of an operand with 32-bit buffer offsets.
  if (dw && t <= 2 && 32 * K < (1ll << 31)) {
    if (t == 1)
      hipLaunchKernelGGL((block_matmul_skinny_staged<AE, BE, 1>), dim3((unsigned)gx),
                         dim3(kSkinnyThreads), 0, stream, a, sa, b, sb, c, M, N, K, accumulate);
    else
      hipLaunchKernelGGL((block_matmul_skinny_staged<AE, BE, 2>), dim3((unsigned)gx),
                         dim3(kSkinnyThreads), 0, stream, a, sa, b, sb, c, M, N, K, accumulate);
    return hipGetLastError();
  }
  if (t == 1)
    hipLaunchKernelGGL((block_matmul_skinny<AE, BE, 1>), grid, dim3(kSkinnyThreads), 0, stream,
                       a, sa, b, sb, c, M, N, K, accumulate, dw);
  else if (t == 2)
    hipLaunchKernelGGL((block_matmul_skinny<AE, BE, 2>), grid, dim3(kSkinnyThreads), 0, stream,
                       a, sa, b, sb, c, M, N, K, accumulate, dw);
  else
    hipLaunchKernelGGL((block_matmul_skinny<AE, BE, 4>), grid, dim3(kSkinnyThreads), 0, stream,
                       a, sa, b, sb, c, M, N, K, accumulate, dw);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fused activation quantize + matmul: C[M,N] (+)= Q(A) . B^T with A float32
// [M, K] and Q the last-axis MX quantize of mx_quantize (same block
// exponent, same element rounding, same codes: the encode of codec_common.h),
// B^T [N, K] block-scaled.  The quantized A never leaves the chip: each K
// stage of 128 loads the tile's float32 A rows, quantizes them in registers
// and writes codes and scale bytes into the LDS stage that the MFMAs read,
// in the layout of the tiled kernel (so its operand reads, the exact split of
// an E4M3 operand against E2M1, and its epilogue apply unchanged).
//
// Tiles of 128 x 256, 8 waves of 64 x 64 (2 x 2 MFMA tiles of 32x32x64), two
// LDS stage buffers; stage st + 1's global loads go out after stage st's
// barrier and land during its MFMAs.  A's rows are read (and quantized) once per tile column,
// i.e. N / 256 times over: the price of not storing Q(A).  (Measured on the
// prefill workload: 128 x 128 tiles 2.78 ms, 128 x 256 1.91 ms, and 1.78 ms
// with the next stage's loads in flight during the MFMAs.)
//
// A loads: wave w covers rows 16w .. 16w + 15 of the tile, two rows per
// 16-byte load instruction (lane l: row 2i + l / 32, floats 4 (l % 32) .. + 3
// of the stage), so one instruction reads two contiguous 512-byte row pieces
// and each aligned group of 8 lanes holds one 32-element block, whose amax is
// reduced across the 8 lanes as in the quantize kernel.
// ---------------------------------------------------------------------------
constexpr int kFusedTM = 128, kFusedTN = 256, kFusedTK = 128;
constexpr int kFusedWN = kFusedTN / 64;                   // waves along N; 2 along M
constexpr int kFusedThreads = 64 * 2 * kFusedWN;
constexpr int kFusedPairs = kFusedTM / (2 * kFusedWN) / 2;  // A row pairs each wave encodes

// Max of v over each aligned group of 8 lanes.
__device__ __forceinline__ uint32_t max_over_8_lanes(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // lane ^ 1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // lane ^ 2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // 7 - lane
  return v;
}

template <int AE, int BE>
struct FusedStage {
  static constexpr int kA = Stage<AE, kFusedTK, 4, kFusedTM>::kBytes;  // A codes
  static constexpr int kB = Stage<BE, kFusedTK, 4, kFusedTN>::kBytes;  // B^T codes
  static constexpr int kBytes = kA + kB + 4 * (kFusedTM + kFusedTN);   // + a scale dword per row
  static constexpr int kBChunks = Stage<BE, kFusedTK>::kChunks;        // 16-byte chunks per row
  static constexpr int kBPieces = kB / 16 / kFusedThreads;             // per thread
};

template <int AE, int BE>
__global__ void __launch_bounds__(kFusedThreads)
block_matmul_quant_a(const float* __restrict__ a, const uint8_t* __restrict__ b,
                     const uint8_t* __restrict__ sb, float* __restrict__ c, int64_t M, int64_t N,
                     int64_t K, int accumulate, int tiles_m, int tiles_n) {
  using FS = FusedStage<AE, BE>;
  using F = codec::Fmt<AE>;
  constexpr int kMQ = 2, kNQ = 2;  // 32x32 MFMA tiles per wave
  __shared__ __attribute__((aligned(1024))) uint8_t smem0[FS::kBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t smem1[FS::kBytes];

  // Tile order as in the tiled kernel: a contiguous range of tiles per XCD,
  // walked in groups of up to 8 tile-rows.
  const int nwg = tiles_m * tiles_n;
  int pid = blockIdx.x;
  if ((nwg & 7) == 0) pid = (pid & 7) * (nwg >> 3) + (pid >> 3);
  constexpr int kGroup = 8;
  const int in_group = kGroup * tiles_n;
  const int first_m = (pid / in_group) * kGroup;
  const int gsize = min(tiles_m - first_m, kGroup);
  const int tm = first_m + (pid % in_group) % gsize;
  const int tn = (pid % in_group) / gsize;
  const int64_t m0 = (int64_t)tm * kFusedTM, n0 = (int64_t)tn * kFusedTN;

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave / kFusedWN, wn = wave % kFusedWN, g = lane >> 5, lr = lane & 31;
  const int64_t kblocks = K / 32;
  const int stages = (int)((K + kFusedTK - 1) / kFusedTK);
  constexpr int kBRowBytes = Stage<BE, kFusedTK>::kRowBytes;      // per stage
  const int64_t b_row_bytes = BE == kE2M1 ? K / 2 : K;
  constexpr int kBChunkK = BE == kE2M1 ? 32 : 16;                 // K elements per chunk

  const int acol = 4 * (lane & 31);  // this lane's first float of a stage row

  // Registers carrying a stage's global loads: B^T's codes (plain 16-byte
  // loads), for t < TN the scale dword of row n0 + t, and this wave's A rows.
  // Stage st + 1's loads are issued right after stage st's barrier, so that
  // they land while stage st's MFMAs run.
  uint4 bv[FS::kBPieces];
  uint32_t bsv = 0;
  float4 av[kFusedPairs];  // row pair i: row 2i + lane / 32 of this wave's rows

  auto load_stage = [&](int st) {
#pragma unroll
    for (int p = 0; p < FS::kBPieces; ++p) {
      const int P = p * kFusedThreads + t;
      const int row = P / FS::kBChunks, ch = P % FS::kBChunks;
      const int64_t grow = n0 + row;
      const bool ok = grow < N && (int64_t)st * kFusedTK + ch * kBChunkK < K;
      bv[p] = ok ? *reinterpret_cast<const uint4*>(b + grow * b_row_bytes +
                                                   (int64_t)st * kBRowBytes + 16 * ch)
                 : make_uint4(0u, 0u, 0u, 0u);
    }
    if (t < kFusedTN) {
      // Blocks past K and rows past N get scale 2^0: their codes are zero, and
      // a 0xFF byte would poison the row in the MFMA.
      uint32_t w = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t kb = 4 * (int64_t)st + j;
        const uint32_t byte = (n0 + t < N && kb < kblocks) ? sb[(n0 + t) * kblocks + kb] : 127u;
        w |= byte << (8 * j);
      }
      bsv = w;
    }
    const int64_t k = (int64_t)st * kFusedTK + acol;
#pragma unroll
    for (int i = 0; i < kFusedPairs; ++i) {
      const int64_t row = min(m0 + 2 * kFusedPairs * wave + 2 * i + (lane >> 5), M - 1);
      av[i] = k < K ? *reinterpret_cast<const float4*>(a + row * K + k)
                    : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };

  // Encode stage st's A rows (already in av) into buf, four row pairs at a
  // time: the block amax over each group of 8 lanes, the encode (the
  // hardware convert unless a live lane of the wave holds a possible
  // midpoint; the results are the same either way), codes and scale bytes;
  // then B^T's codes and scales.
  auto store_stage = [&](int st, uint8_t* buf) {
    const int64_t k = (int64_t)st * kFusedTK + acol;
#pragma unroll
    for (int c = 0; c < kFusedPairs / 4; ++c) {
      uint32_t amax[4], low = 0xFFFFFFFFu;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 v = av[4 * c + j];
        const uint32_t b0 = __float_as_uint(v.x), b1 = __float_as_uint(v.y);
        const uint32_t b2 = __float_as_uint(v.z), b3 = __float_as_uint(v.w);
        amax[j] = max(max(b0 & 0x7FFFFFFFu, b1 & 0x7FFFFFFFu),
                      max(b2 & 0x7FFFFFFFu, b3 & 0x7FFFFFFFu));
        if (k < K && m0 + 2 * kFusedPairs * wave + 2 * (4 * c + j) + (lane >> 5) < M)
          low = min(low, min(min(b0 << F::kTieShift, b1 << F::kTieShift),
                             min(b2 << F::kTieShift, b3 << F::kTieShift)));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) amax[j] = max_over_8_lanes(amax[j]);
      bool exact = low == 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) exact |= amax[j] < 0x0D800000u;
      const bool fast = __ballot(exact) == 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 2 * kFusedPairs * wave + 2 * (4 * c + j) + (lane >> 5);  // row in the tile
        const int e = codec::block_exponent<AE>(amax[j]);
        const bool nonfinite = amax[j] >= 0x7F800000u;
        const uint32_t byte = amax[j] == 0 ? 127u : (nonfinite ? 0xFFu : (uint32_t)(e + 127));
        const float scale = __uint_as_float((uint32_t)max(e + 127, 1) << 23);
        const float inv_scale = __uint_as_float((uint32_t)(127 - e) << 23);
        const float4 v = av[4 * c + j];
        uint32_t w = fast ? codec::convert4<AE>(v, scale, AE == kE4M3 ? 448.0f * scale : 0.0f)
                          : codec::round4<AE>(v, inv_scale);
        w = nonfinite ? 0u : w;
        if (AE == kE4M3)
          *reinterpret_cast<uint32_t*>(buf + lds_off<AE, kFusedTK>(r, acol >> 4) + (acol & 15)) = w;
        else
          *reinterpret_cast<uint16_t*>(buf + lds_off<AE, kFusedTK>(r, acol >> 5) +
                                       ((acol >> 1) & 15)) = (uint16_t)w;
        if ((lane & 7) == 0) buf[FS::kA + FS::kB + 4 * r + ((lane & 31) >> 3)] = (uint8_t)byte;
      }
    }
#pragma unroll
    for (int p = 0; p < FS::kBPieces; ++p) {
      const int P = p * kFusedThreads + t;
      *reinterpret_cast<uint4*>(buf + FS::kA +
                                lds_off<BE, kFusedTK>(P / FS::kBChunks, P % FS::kBChunks)) = bv[p];
    }
    if (t < kFusedTN) reinterpret_cast<uint32_t*>(buf + FS::kA + FS::kB)[kFusedTM + t] = bsv;
  };

  v16f acc[kMQ][kNQ];
#pragma unroll
  for (int i = 0; i < kMQ; ++i)
#pragma unroll
    for (int j = 0; j < kNQ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  const int ar = wm * 64 + lr, br = wn * 64 + lr;

  auto mfma = [&](const uint8_t* buf) {
    const uint8_t* la = buf;
    const uint8_t* lb = buf + FS::kA;
    const uint32_t* lsa = reinterpret_cast<const uint32_t*>(buf + FS::kA + FS::kB);
    const uint32_t* lsb = lsa + kFusedTM;
    int sas[kMQ], sbs[kNQ];
#pragma unroll
    for (int i = 0; i < kMQ; ++i) sas[i] = (int)(lsa[ar + 32 * i] >> (8 * g));
#pragma unroll
    for (int q = 0; q < kNQ; ++q) sbs[q] = (int)(lsb[br + 32 * q] >> (8 * g));
    constexpr int fa = Operand<AE>::kFmt, fb = Operand<BE>::kFmt;
    auto kstep = [&](auto H) {
      constexpr int h = decltype(H)::value;
      v8i af[kMQ], bf[kNQ];
#pragma unroll
      for (int i = 0; i < kMQ; ++i) af[i] = read_operand<AE, kFusedTK>(la, ar + 32 * i, h, g);
#pragma unroll
      for (int q = 0; q < kNQ; ++q) bf[q] = read_operand<BE, kFusedTK>(lb, br + 32 * q, h, g);
      constexpr int sel = 2 * h;  // byte 2h of the shifted dword: block 2h + g of the stage
#pragma unroll
      for (int i = 0; i < kMQ; ++i)
#pragma unroll
        for (int q = 0; q < kNQ; ++q) {
          if constexpr (Split<AE, BE>::kA) {
            const v8i ah = e4m3_high(af[i]);
            acc[i][q] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                ah, bf[q], acc[i][q], fa, fb, sel, sas[i], sel, sbs[q]);
            acc[i][q] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                af[i] ^ ah, bf[q], acc[i][q], fa, fb, sel, sas[i], sel, sbs[q]);
          } else if constexpr (Split<AE, BE>::kB) {
            const v8i bh = e4m3_high(bf[q]);
            acc[i][q] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                af[i], bh, acc[i][q], fa, fb, sel, sas[i], sel, sbs[q]);
            acc[i][q] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                af[i], bf[q] ^ bh, acc[i][q], fa, fb, sel, sas[i], sel, sbs[q]);
          } else {
            acc[i][q] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                af[i], bf[q], acc[i][q], fa, fb, sel, sas[i], sel, sbs[q]);
          }
        }
    };
    static_assert(kFusedTK == 128, "two MFMA K steps per stage");
    kstep(std::integral_constant<int, 0>{});
    kstep(std::integral_constant<int, 1>{});
  };

  // One barrier per stage: it follows this stage's LDS writes and every
  // wave's MFMAs of the previous stage, whose buffer the next stage rewrites.
  load_stage(0);
  for (int st = 0; st < stages; ++st) {
    uint8_t* buf = (st & 1) ? smem1 : smem0;
    store_stage(st, buf);
    __syncthreads();
    if (st + 1 < stages) load_stage(st + 1);
    mfma(buf);
  }

  // Epilogue as in the tiled kernel: lane holds C[8(e/4) + 4g + (e%4)][lr] of
  // each 32x32 tile.
#pragma unroll
  for (int i = 0; i < kMQ; ++i)
#pragma unroll
    for (int q = 0; q < kNQ; ++q) {
      const int64_t col = n0 + wn * 64 + 32 * q + lr;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = m0 + wm * 64 + 32 * i + 8 * (e >> 2) + 4 * g + (e & 3);
        if (row < M && col < N) {
          float v = acc[i][q][e];
          if (accumulate) v += c[row * N + col];
          __builtin_nontemporal_store(v, c + row * N + col);
        }
      }
    }
}

template <int AE, int BE>
hipError_t launch_quant_a_typed(const float* a, const uint8_t* b, const uint8_t* sb, float* c,
                                int64_t M, int64_t N, int64_t K, int accumulate,
                                hipStream_t stream) {
  const int64_t tiles_m = (M + kFusedTM - 1) / kFusedTM, tiles_n = (N + kFusedTN - 1) / kFusedTN;
  if (tiles_m * tiles_n > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((block_matmul_quant_a<AE, BE>), dim3((unsigned)(tiles_m * tiles_n)),
                     dim3(kFusedThreads), 0, stream, a, b, sb, c, M, N, K, accumulate,
                     (int)tiles_m, (int)tiles_n);
  return hipGetLastError();
}

template <int AE, int BE>
hipError_t launch_typed(const uint8_t* a, const uint8_t* sa, const uint8_t* b,
                        const uint8_t* sb, float* c, int64_t M, int64_t N, int64_t K,
                        int accumulate, hipStream_t stream) {
  // The tiled kernel addresses a 256-row slab of either operand with 32-bit
  // buffer offsets, and stages scales either as aligned 16-byte row slices
  // (16 blocks; K % 512 == 0, 16-byte aligned scale arrays) or as one dword
  // per row and 128-K stage (K % 128 == 0, 4-byte aligned scale arrays).
  const int64_t slab_a = 256 * (AE == kE2M1 ? K / 2 : K), slab_b = 256 * (BE == kE2M1 ? K / 2 : K);
  const uintptr_t align = reinterpret_cast<uintptr_t>(sa) | reinterpret_cast<uintptr_t>(sb);
  const bool tiled = M > 64 && slab_a < (1ll << 31) && slab_b < (1ll << 31) &&
                     M * (K / 32) < (1ll << 31) && N * (K / 32) < (1ll << 31);
  if (tiled && K % 512 == 0 && (align & 15) == 0)
    return launch_tiled_split<AE, BE, false>(a, sa, b, sb, c, M, N, K, accumulate, stream);
  if (tiled && K % 128 == 0 && (align & 3) == 0)
    return launch_tiled_split<AE, BE, true>(a, sa, b, sb, c, M, N, K, accumulate, stream);
  return launch_skinny<AE, BE>(a, sa, b, sb, c, M, N, K, accumulate, stream);
}

}  // namespace

hipError_t launch_block_matmul_quant_a(const float* a, int a_elem, const void* b_codes,
                                       const uint8_t* b_scales, int b_elem, float* c, int64_t M,
                                       int64_t N, int64_t K, int accumulate, hipStream_t stream) {
  const uint8_t* b = static_cast<const uint8_t*>(b_codes);
  if (a_elem == kE2M1 && b_elem == kE2M1)
    return launch_quant_a_typed<kE2M1, kE2M1>(a, b, b_scales, c, M, N, K, accumulate, stream);
  if (a_elem == kE2M1 && b_elem == kE4M3)
    return launch_quant_a_typed<kE2M1, kE4M3>(a, b, b_scales, c, M, N, K, accumulate, stream);
  if (a_elem == kE4M3 && b_elem == kE2M1)
    return launch_quant_a_typed<kE4M3, kE2M1>(a, b, b_scales, c, M, N, K, accumulate, stream);
  return launch_quant_a_typed<kE4M3, kE4M3>(a, b, b_scales, c, M, N, K, accumulate, stream);
}

hipError_t launch_block_matmul(const void* a_codes, const uint8_t* a_scales, int a_elem,
                               const void* b_codes, const uint8_t* b_scales, int b_elem,
                               float* c, int64_t M, int64_t N, int64_t K, int accumulate,
                               hipStream_t stream) {
  const uint8_t* a = static_cast<const uint8_t*>(a_codes);
  const uint8_t* b = static_cast<const uint8_t*>(b_codes);
  if (a_elem == kE2M1 && b_elem == kE2M1)
    return launch_typed<kE2M1, kE2M1>(a, a_scales, b, b_scales, c, M, N, K, accumulate, stream);
  if (a_elem == kE2M1 && b_elem == kE4M3)
    return launch_typed<kE2M1, kE4M3>(a, a_scales, b, b_scales, c, M, N, K, accumulate, stream);
  if (a_elem == kE4M3 && b_elem == kE2M1)
    return launch_typed<kE4M3, kE2M1>(a, a_scales, b, b_scales, c, M, N, K, accumulate, stream);
  return launch_typed<kE4M3, kE4M3>(a, a_scales, b, b_scales, c, M, N, K, accumulate, stream);
}

}  // namespace mx
