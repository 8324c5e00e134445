// MX block matmul: C[M,N] (+)= A[M,K] . B[K,N], A and B^T [N,K] block-scaled
// along K, on CDNA4's block-scaled MFMA (v_mfma_scale_f32_16x16x128_f8f6f4).
//
// Semantics: the dialect page "A Dialect Is a Set of Co-Designed Decisions",
// sections "The four ops" (block_matmul, C += A.B) and "The block axis" (the
// scale of A[m,k] is S[m, k/32], constant along each 32-run of the reduction,
// so it multiplies that run's partial sum).  The hardware instruction takes
// exactly that form: per lane, 32 consecutive K elements of one row (one MX
// block) and that block's E8M0 scale byte.
//
// Operand layout of the 16x16x128 instruction (wave64), established with
// one-hot probes on gfx950 (lane group g = l / 16, row = l % 16):
//   * FP4 operands fill the first 4 VGPRs: lane l holds the 32 K elements
//     [32g, 32g+32) of its row, element 2i in the low nibble of byte i -- the
//     packing of the codes in memory, so one 16-byte load fills them.
//   * FP8 operands fill 8 VGPRs: bytes 0..15 hold K [16g, 16g+16) and bytes
//     16..31 hold K [64+16g, 64+16g+16) of the row.
//   * The scale operand of lane l is the E8M0 byte of block g (K [32g, 32g+32))
//     of its row, for either element format.
//   * Output: lane l holds C[4g + j][l % 16] in accumulator j = 0..3.
// B^T rows use the same layout as A rows (B column n = B^T row n).
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

template <int AE, int BE>
hipError_t launch_typed(const uint8_t* a, const uint8_t* sa, const uint8_t* b,
                        const uint8_t* sb, float* c, int64_t M, int64_t N, int64_t K,
                        int accumulate, hipStream_t stream) {
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
