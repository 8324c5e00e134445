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

// One wave computes one 16x16 tile of C.
template <int AE, int BE>
__global__ void __launch_bounds__(256)
block_matmul_simple(const uint8_t* __restrict__ a, const uint8_t* __restrict__ sa,
                    const uint8_t* __restrict__ b, const uint8_t* __restrict__ sb,
                    float* __restrict__ c, int64_t M, int64_t N, int64_t K, int accumulate) {
  const int lane = threadIdx.x & 63;
  const int64_t tile = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
  const int64_t tiles_n = (N + 15) / 16;
  const int64_t tiles = ((M + 15) / 16) * tiles_n;
  if (tile >= tiles) return;
  const int64_t m0 = (tile / tiles_n) * 16, n0 = (tile % tiles_n) * 16;
  const int64_t kblocks = K / 32;
  const int64_t arow = m0 + (lane & 15), brow = n0 + (lane & 15);
  const int kq = lane >> 4;

  v4f acc = {0.f, 0.f, 0.f, 0.f};
  for (int64_t kb0 = 0; kb0 < kblocks; kb0 += 4) {
    const int64_t kb = kb0 + kq;
    const v8i av = load_operand<AE>(a, arow, M, kb0 * 32, kq, K);
    const v8i bv = load_operand<BE>(b, brow, N, kb0 * 32, kq, K);
    const int as = load_scale(sa, arow, M, kb, kblocks);
    const int bs = load_scale(sb, brow, N, kb, kblocks);
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, Operand<AE>::kFmt,
                                                           Operand<BE>::kFmt, 0, as, 0, bs);
  }
  const int64_t col = n0 + (lane & 15);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t row = m0 + 4 * kq + j;
    if (row < M && col < N) {
      float v = acc[j];
      if (accumulate) v += c[row * N + col];
      c[row * N + col] = v;
    }
  }
}

// ---------------------------------------------------------------------------
// Tiled kernel: 256x256 output tile per workgroup of 4 waves (2 x 2), each
// wave 128x128 = 4 x 4 tiles of the 32x32x64 scaled MFMA.  K advances in
// stages of 128 elements: codes are staged in LDS (double-buffered, the next
// stage prefetched into registers while the current one feeds the MFMAs) and
// the scale bytes go straight from global memory to registers.
// ---------------------------------------------------------------------------
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kTM = 256, kTN = 256, kTK = 128, kTThreads = 256;

template <int ELEM>
struct Stage {
  static constexpr int kRowBytes = ELEM == kE2M1 ? kTK / 2 : kTK;  // 64 or 128
  static constexpr int kChunks = kRowBytes / 16;                     // 16-B chunks per row
  static constexpr int kBytes = 256 * kRowBytes;                     // one 256-row tile
  static constexpr int kLoads = 256 * kChunks / kTThreads;           // chunks per thread
  static constexpr int kRowStep = kTThreads / kChunks;               // rows between a thread's chunks
};

// LDS byte offset of 16-byte chunk c of row r of a staged tile.  Rows are
// packed into 128-byte lines (one FP8 row or two FP4 rows per line) and the
// chunk index within the line is XOR-swizzled with the line index, so that
// eight lanes touching the same logical chunk of eight consecutive rows (an
// MFMA operand read) or eight consecutive chunks (a staging write) address
// eight different 16-byte bank groups.
template <int ELEM>
__device__ __forceinline__ int lds_off(int r, int c) {
  if (ELEM == kE4M3) return r * 128 + ((c ^ (r & 7)) << 4);
  const int line = r >> 1;
  const int q = ((r & 1) << 2) | c;
  return line * 128 + ((q ^ (line & 7)) << 4);
}

// Buffer resource over `bytes` bytes at `base` (raw buffer: offsets are byte
// offsets; loads at offsets past `bytes` return zeros).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

constexpr uint32_t kOutOfRange = 0x80000000u;  // past every resource used here

// Stage one 256-row tile of codes straight into LDS with buffer loads that
// write LDS directly (each wave instruction fills 1 KiB: lane i writes bytes
// [16i, 16i+16) of it).  LDS position (line L, chunk p) must hold logical
// chunk p ^ (L & 7) of its row (the swizzle of lds_off), so each lane fetches
// that chunk from global memory.  Within one instruction, lane i covers line
// 8j' + i/8 (j' = the instruction's index in the tile), so its row offset
// inside the instruction and its chunk do not depend on j'.
template <int ELEM>
struct Stager {
  static constexpr int kInstr = Stage<ELEM>::kBytes / 1024 / 4;    // per wave
  static constexpr int kRowsPerInstr = ELEM == kE4M3 ? 8 : 16;
  uint32_t lane_off;   // row-in-instruction * row_bytes + 16 * chunk
  uint32_t chunk16;    // 16 * chunk: byte of the chunk within the stage's row slice
  uint32_t instr_step; // bytes between consecutive instructions' first rows

  __device__ __forceinline__ Stager(uint32_t row_bytes, int lane) {
    const int p = lane & 7, l8 = lane >> 3;
    const int q = p ^ l8;
    int r, c;
    if (ELEM == kE4M3) {
      r = l8;
      c = q;
    } else {
      r = 2 * l8 + (q >> 2);
      c = q & 3;
    }
    chunk16 = 16u * c;
    lane_off = (uint32_t)r * row_bytes + chunk16;
    instr_step = kRowsPerInstr * row_bytes;
  }

  // `rsrc` starts at the tile's first row and ends at the matrix's last row,
  // so rows past the matrix read as zeros; chunks past K (only in a last,
  // partial stage) are sent out of range and read as zeros too.
  __device__ __forceinline__ void load(uint8_t* lds_tile, __amdgpu_buffer_rsrc_t rsrc,
                                       uint32_t row_bytes, uint32_t byte0, int wave) const {
    const bool in_k = byte0 + chunk16 < row_bytes;
#pragma unroll
    for (int j = 0; j < kInstr; ++j) {
      const int ji = wave * kInstr + j;
      const uint32_t off = in_k ? lane_off + ji * instr_step : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc, (__attribute__((address_space(3))) void*)(lds_tile + ji * 1024), 16, off, byte0,
          0, 0);
    }
  }
};

// MFMA operand of row r for K sub-step ks (64 elements) of the staged tile.
template <int ELEM>
__device__ __forceinline__ v8i read_operand(const uint8_t* lds, int r, int ks, int g) {
  if (ELEM == kE4M3) {
    const v4i lo = *reinterpret_cast<const v4i*>(lds + lds_off<ELEM>(r, 4 * ks + g));
    const v4i hi = *reinterpret_cast<const v4i*>(lds + lds_off<ELEM>(r, 4 * ks + 2 + g));
    return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  } else {
    const v4i lo = *reinterpret_cast<const v4i*>(lds + lds_off<ELEM>(r, 2 * ks + g));
    return v8i{lo.x, lo.y, lo.z, lo.w, 0, 0, 0, 0};
  }
}

// The four scale bytes of blocks [kb0, kb0+4) of row r of a tile, from a
// buffer resource over the tile's scale rows.  Bytes past the resource (rows
// past the matrix) and blocks past K read as 0 -- a finite scale (2^-127)
// multiplying zero codes.  DWORD: one 4-byte load (row stride and base are
// 4-byte aligned); otherwise four byte loads.
template <bool DWORD>
__device__ __forceinline__ uint32_t load_scales4(__amdgpu_buffer_rsrc_t rs, int r,
                                                 int64_t kblocks, int64_t kb0) {
  const uint32_t base = (uint32_t)(r * kblocks + kb0);
  if (DWORD) return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, base, 0, 0);
  uint32_t v = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t off = kb0 + j < kblocks ? base + j : kOutOfRange;
    v |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rs, off, 0, 0) << (8 * j);
  }
  return v;
}

template <int AE, int BE, int KS>
__device__ __forceinline__ void mfma_substep(v16f (&acc)[4][4], const uint8_t* la,
                                             const uint8_t* lb, int arow0, int brow0, int lr,
                                             int g, const uint32_t (&sa)[4],
                                             const uint32_t (&sb)[4]) {
  v8i af[4], bf[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) af[i] = read_operand<AE>(la, arow0 + 32 * i + lr, KS, g);
#pragma unroll
  for (int j = 0; j < 4; ++j) bf[j] = read_operand<BE>(lb, brow0 + 32 * j + lr, KS, g);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          af[i], bf[j], acc[i][j], Operand<AE>::kFmt, Operand<BE>::kFmt, 2 * KS, (int)sa[i],
          2 * KS, (int)sb[j]);
}

template <int AE, int BE, bool SDW>
__global__ void __launch_bounds__(kTThreads)
block_matmul_tiled(const uint8_t* __restrict__ a, const uint8_t* __restrict__ sa,
                   const uint8_t* __restrict__ b, const uint8_t* __restrict__ sb,
                   float* __restrict__ c, int64_t M, int64_t N, int64_t K, int accumulate,
                   int tiles_m, int tiles_n) {
  constexpr int kA = Stage<AE>::kBytes, kB = Stage<BE>::kBytes;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * (kA + kB)];

  // Tile order: the hardware deals workgroups round-robin to the 8 XCDs, so
  // give each XCD a contiguous range of tiles, walked in groups of up to 8
  // tile-rows so that concurrently running tiles share A rows and B columns
  // in that XCD's L2.
  const int nwg = tiles_m * tiles_n;
  int pid = blockIdx.x;
  if ((nwg & 7) == 0) pid = (pid & 7) * (nwg >> 3) + (pid >> 3);
  constexpr int kGroup = 8;
  const int in_group = kGroup * tiles_n;
  const int first_m = (pid / in_group) * kGroup;
  const int gsize = min(tiles_m - first_m, kGroup);
  const int tm = first_m + (pid % in_group) % gsize;
  const int tn = (pid % in_group) / gsize;
  const int64_t m0 = (int64_t)tm * kTM, n0 = (int64_t)tn * kTN;

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 1, wn = wave & 1, g = lane >> 5, lr = lane & 31;
  const uint32_t a_row_bytes = (uint32_t)(AE == kE2M1 ? K / 2 : K);
  const uint32_t b_row_bytes = (uint32_t)(BE == kE2M1 ? K / 2 : K);
  const Stager<AE> stage_a(a_row_bytes, lane);
  const Stager<BE> stage_b(b_row_bytes, lane);
  const int64_t kblocks = K / 32;
  const int nstages = (int)((K + kTK - 1) / kTK);
  const int64_t rows_a = min(M - m0, (int64_t)kTM), rows_b = min(N - n0, (int64_t)kTN);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a + m0 * a_row_bytes, rows_a * a_row_bytes);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(b + n0 * b_row_bytes, rows_b * b_row_bytes);
  // (a 256-row slab of either operand is below 2^31 bytes: checked at launch)
  const __amdgpu_buffer_rsrc_t rsa = make_rsrc(sa + m0 * kblocks, rows_a * kblocks);
  const __amdgpu_buffer_rsrc_t rsb = make_rsrc(sb + n0 * kblocks, rows_b * kblocks);
  const int ar = wm * 128 + lr, br = wn * 128 + lr;  // this lane's first A / B^T tile row

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  uint32_t sac[4], sbc[4], san[4], sbn[4];
  stage_a.load(smem, ra, a_row_bytes, 0, wave);
  stage_b.load(smem + kA, rb, b_row_bytes, 0, wave);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    san[i] = load_scales4<SDW>(rsa, ar + 32 * i, kblocks, 0);
    sbn[i] = load_scales4<SDW>(rsb, br + 32 * i, kblocks, 0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int st = 0; st < nstages; ++st) {
    // Scales of this stage, shifted so that byte 0 / byte 2 hold this lane's
    // block of K sub-step 0 / 1 (lane group g takes block g of each sub-step).
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sac[i] = san[i] >> (8 * g);
      sbc[i] = sbn[i] >> (8 * g);
    }
    const uint8_t* cur = smem + (st & 1) * (kA + kB);
    uint8_t* nxt = smem + ((st + 1) & 1) * (kA + kB);
    if (st + 1 < nstages) {
      stage_a.load(nxt, ra, a_row_bytes, (uint32_t)(st + 1) * Stage<AE>::kRowBytes, wave);
      stage_b.load(nxt + kA, rb, b_row_bytes, (uint32_t)(st + 1) * Stage<BE>::kRowBytes, wave);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        san[i] = load_scales4<SDW>(rsa, ar + 32 * i, kblocks, 4 * (st + 1));
        sbn[i] = load_scales4<SDW>(rsb, br + 32 * i, kblocks, 4 * (st + 1));
      }
    }
    mfma_substep<AE, BE, 0>(acc, cur, cur + kA, wm * 128, wn * 128, lr, g, sac, sbc);
    mfma_substep<AE, BE, 1>(acc, cur, cur + kA, wm * 128, wn * 128, lr, g, sac, sbc);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // Epilogue: lane holds C[8(e/4) + 4g + (e%4)][lr] of each 32x32 tile.
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = n0 + wn * 128 + 32 * j + lr;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = m0 + wm * 128 + 32 * i + 8 * (e >> 2) + 4 * g + (e & 3);
        if (row < M && col < N) {
          float v = acc[i][j][e];
          if (accumulate) v += c[row * N + col];
          c[row * N + col] = v;
        }
      }
    }
}

template <int AE, int BE>
hipError_t launch_tiled(const uint8_t* a, const uint8_t* sa, const uint8_t* b, const uint8_t* sb,
                        float* c, int64_t M, int64_t N, int64_t K, int accumulate,
                        hipStream_t stream) {
  const int64_t tiles_m = (M + kTM - 1) / kTM, tiles_n = (N + kTN - 1) / kTN;
  const int64_t kblocks = K / 32;
  const bool dw = (kblocks % 4 == 0) && ((reinterpret_cast<uintptr_t>(sa) & 3) == 0) &&
                  ((reinterpret_cast<uintptr_t>(sb) & 3) == 0);
  const dim3 grid((unsigned)(tiles_m * tiles_n)), block(kTThreads);
  if (dw)
    hipLaunchKernelGGL((block_matmul_tiled<AE, BE, true>), grid, block, 0, stream, a, sa, b, sb,
                       c, M, N, K, accumulate, (int)tiles_m, (int)tiles_n);
  else
    hipLaunchKernelGGL((block_matmul_tiled<AE, BE, false>), grid, block, 0, stream, a, sa, b,
                       sb, c, M, N, K, accumulate, (int)tiles_m, (int)tiles_n);
  return hipGetLastError();
}

template <int AE, int BE>
hipError_t launch_typed(const uint8_t* a, const uint8_t* sa, const uint8_t* b,
                        const uint8_t* sb, float* c, int64_t M, int64_t N, int64_t K,
                        int accumulate, hipStream_t stream) {
  // The tiled kernel addresses a 256-row slab of either operand with 32-bit
  // buffer offsets.
  const int64_t slab_a = 256 * (AE == kE2M1 ? K / 2 : K), slab_b = 256 * (BE == kE2M1 ? K / 2 : K);
  if (M > 64 && slab_a < (1ll << 31) && slab_b < (1ll << 31))
    return launch_tiled<AE, BE>(a, sa, b, sb, c, M, N, K, accumulate, stream);
  const int64_t tiles = ((M + 15) / 16) * ((N + 15) / 16);
  const int64_t grid = (tiles + 3) / 4;
  hipLaunchKernelGGL((block_matmul_simple<AE, BE>), dim3((unsigned)grid), dim3(256), 0, stream,
                     a, sa, b, sb, c, M, N, K, accumulate);
  return hipGetLastError();
}

}  // namespace

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
