// Internal declarations shared by the libmx host layer and its HIP kernels.
// Not part of the public interface (that is include/libmx.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

// Element formats, numbered as in the public header.
enum Elem : int { kE2M1 = 1, kE4M3 = 2 };

// Streaming codec kernels (quantize.hip, dequantize.hip).  n_blocks is
// rows*cols/32; buffers are dense and 16-byte aligned.
hipError_t launch_quantize(const float* x, void* codes, uint8_t* scales, int64_t n_blocks,
                           int elem, hipStream_t stream);
hipError_t launch_dequantize(const void* codes, const uint8_t* scales, float* y,
                             int64_t n_blocks, int elem, hipStream_t stream);

// Codec with blocks along axis 0, block-major storage (codec_axis0.hip);
// rows % 32 == 0.
hipError_t launch_quantize_axis0(const float* x, void* codes, uint8_t* scales, int64_t rows,
                                 int64_t cols, int elem, hipStream_t stream);
hipError_t launch_dequantize_axis0(const void* codes, const uint8_t* scales, float* y,
                                   int64_t rows, int64_t cols, int elem, hipStream_t stream);

// scales[i] -> scales of 2^j times the tensor, in place (scale_ops.hip).
hipError_t launch_fold_scale(uint8_t* scales, int64_t n, int j, hipStream_t stream);

// Block-scaled matmul (block_matmul.hip).  C[M,N] (+)= A[M,K] . (B^T[N,K])^T.
hipError_t launch_block_matmul(const void* a_codes, const uint8_t* a_scales, int a_elem,
                               const void* b_codes, const uint8_t* b_scales, int b_elem,
                               float* c, int64_t M, int64_t N, int64_t K, int accumulate,
                               hipStream_t stream);

// Float32 A [M, K] quantized along K in the matmul's prologue, times block-
// scaled B^T [N, K] (block_matmul.hip).  a is 16-byte aligned, K % 32 == 0.
hipError_t launch_block_matmul_quant_a(const float* a, int a_elem, const void* b_codes,
                                       const uint8_t* b_scales, int b_elem, float* c, int64_t M,
                                       int64_t N, int64_t K, int accumulate, hipStream_t stream);

// Block-scaled A times float32 B[K, N] (block_matmul_f32b.hip).
hipError_t launch_block_matmul_f32b(const void* a_codes, const uint8_t* a_scales, int a_elem,
                                    const float* b, float* c, int64_t M, int64_t N, int64_t K,
                                    int accumulate, hipStream_t stream);

}  // namespace mx
