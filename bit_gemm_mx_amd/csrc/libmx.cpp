// libmx C ABI: argument validation and dispatch to the HIP kernels.
//
// Validation mirrors the structural verifier of the dialect page ("A Dialect
// Is a Set of Co-Designed Decisions", section "The type: !mx.tensor": the
// block size is positive and divides the last dimension) plus what the
// kernels need (non-null, 16-byte aligned buffers).  It never looks at data
// and runs before anything is enqueued, so an error leaves every buffer
// untouched.  There is no fallback path: a launch failure is reported.
#include "../../include/libmx.h"

#include <hip/hip_runtime.h>

#include "mx_internal.h"

namespace {

bool is_elem(mx_elem_t e) { return e == MX_E2M1 || e == MX_E4M3; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

mx_status_t check_codec(const void* dense, const void* codes, const uint8_t* scales,
                        int64_t rows, int64_t cols, mx_elem_t elem, int32_t block_size) {
  if (!dense || !codes || !scales) return MX_ERR_NULL;
  if (!is_elem(elem) || block_size != MX_BLOCK_SIZE) return MX_ERR_UNSUPPORTED;
  if (rows < 1 || cols < 1 || cols % MX_BLOCK_SIZE != 0) return MX_ERR_SHAPE;
  if (rows > INT64_MAX / cols) return MX_ERR_SHAPE;
  if (!aligned16(dense) || !aligned16(codes)) return MX_ERR_ALIGN;
  return MX_OK;
}

mx_status_t from_hip(hipError_t e) { return e == hipSuccess ? MX_OK : MX_ERR_HIP; }

}  // namespace

extern "C" {

mx_status_t mx_quantize(const float* x, void* codes, uint8_t* scales, int64_t rows, int64_t cols,
                        mx_elem_t elem, int32_t block_size, mx_stream_t stream) {
  const mx_status_t s = check_codec(x, codes, scales, rows, cols, elem, block_size);
  if (s != MX_OK) return s;
  return from_hip(mx::launch_quantize(x, codes, scales, rows * cols / MX_BLOCK_SIZE, (int)elem,
                                      reinterpret_cast<hipStream_t>(stream)));
}

mx_status_t mx_dequantize(const void* codes, const uint8_t* scales, float* y, int64_t rows,
                          int64_t cols, mx_elem_t elem, int32_t block_size, mx_stream_t stream) {
  const mx_status_t s = check_codec(y, codes, scales, rows, cols, elem, block_size);
  if (s != MX_OK) return s;
  return from_hip(mx::launch_dequantize(codes, scales, y, rows * cols / MX_BLOCK_SIZE, (int)elem,
                                        reinterpret_cast<hipStream_t>(stream)));
}

mx_status_t mx_block_matmul(const void* a_codes, const uint8_t* a_scales, mx_elem_t a_elem,
                            const void* b_codes, const uint8_t* b_scales, mx_elem_t b_elem,
                            float* c, int64_t M, int64_t N, int64_t K, int32_t block_size,
                            int32_t accumulate, mx_stream_t stream) {
  if (!a_codes || !a_scales || !b_codes || !b_scales || !c) return MX_ERR_NULL;
  if (!is_elem(a_elem) || !is_elem(b_elem) || block_size != MX_BLOCK_SIZE)
    return MX_ERR_UNSUPPORTED;
  if (M < 1 || N < 1 || K < 1 || K % MX_BLOCK_SIZE != 0) return MX_ERR_SHAPE;
  if (M > INT64_MAX / K || N > INT64_MAX / K || M > INT64_MAX / N) return MX_ERR_SHAPE;
  if (!aligned16(a_codes) || !aligned16(b_codes) || !aligned16(c)) return MX_ERR_ALIGN;
  return from_hip(mx::launch_block_matmul(a_codes, a_scales, (int)a_elem, b_codes, b_scales,
                                          (int)b_elem, c, M, N, K, accumulate ? 1 : 0,
                                          reinterpret_cast<hipStream_t>(stream)));
}

mx_status_t mx_block_matmul_f32b(const void* a_codes, const uint8_t* a_scales, mx_elem_t a_elem,
                                 const float* b, float* c, int64_t M, int64_t N, int64_t K,
                                 int32_t block_size, int32_t accumulate, mx_stream_t stream) {
  if (!a_codes || !a_scales || !b || !c) return MX_ERR_NULL;
  if (!is_elem(a_elem) || block_size != MX_BLOCK_SIZE) return MX_ERR_UNSUPPORTED;
  if (M < 1 || N < 1 || K < 1 || K % MX_BLOCK_SIZE != 0) return MX_ERR_SHAPE;
  if (M > INT64_MAX / K || N > INT64_MAX / K || M > INT64_MAX / N) return MX_ERR_SHAPE;
  if (!aligned16(a_codes) || (reinterpret_cast<uintptr_t>(b) & 3) ||
      (reinterpret_cast<uintptr_t>(c) & 3))
    return MX_ERR_ALIGN;
  return from_hip(mx::launch_block_matmul_f32b(a_codes, a_scales, (int)a_elem, b, c, M, N, K,
                                               accumulate ? 1 : 0,
                                               reinterpret_cast<hipStream_t>(stream)));
}

mx_status_t mx_block_matmul_quantize_a(const float* a, mx_elem_t a_elem, const void* b_codes,
                                       const uint8_t* b_scales, mx_elem_t b_elem, float* c,
                                       int64_t M, int64_t N, int64_t K, int32_t block_size,
                                       int32_t accumulate, mx_stream_t stream) {
  if (!a || !b_codes || !b_scales || !c) return MX_ERR_NULL;
  if (!is_elem(a_elem) || !is_elem(b_elem) || block_size != MX_BLOCK_SIZE)
    return MX_ERR_UNSUPPORTED;
  if (M < 1 || N < 1 || K < 1 || K % MX_BLOCK_SIZE != 0) return MX_ERR_SHAPE;
  if (M > INT64_MAX / K || N > INT64_MAX / K || M > INT64_MAX / N) return MX_ERR_SHAPE;
  if (!aligned16(a) || !aligned16(b_codes) || (reinterpret_cast<uintptr_t>(c) & 3))
    return MX_ERR_ALIGN;
  return from_hip(mx::launch_block_matmul_quant_a(a, (int)a_elem, b_codes, b_scales, (int)b_elem,
                                                  c, M, N, K, accumulate ? 1 : 0,
                                                  reinterpret_cast<hipStream_t>(stream)));
}

mx_status_t mx_quantize_axis(const float* x, void* codes, uint8_t* scales, int64_t rows,
                             int64_t cols, int32_t axis, mx_elem_t elem, int32_t block_size,
                             mx_stream_t stream) {
  if (axis == 1) return mx_quantize(x, codes, scales, rows, cols, elem, block_size, stream);
  if (axis != 0) return MX_ERR_UNSUPPORTED;
  // Blocks along axis 0 are the blocks of the transposed [cols, rows] matrix.
  const mx_status_t s = check_codec(x, codes, scales, cols, rows, elem, block_size);
  if (s != MX_OK) return s;
  return from_hip(mx::launch_quantize_axis0(x, codes, scales, rows, cols, (int)elem,
                                            reinterpret_cast<hipStream_t>(stream)));
}

mx_status_t mx_dequantize_axis(const void* codes, const uint8_t* scales, float* y, int64_t rows,
                               int64_t cols, int32_t axis, mx_elem_t elem, int32_t block_size,
                               mx_stream_t stream) {
  if (axis == 1) return mx_dequantize(codes, scales, y, rows, cols, elem, block_size, stream);
  if (axis != 0) return MX_ERR_UNSUPPORTED;
  const mx_status_t s = check_codec(y, codes, scales, cols, rows, elem, block_size);
  if (s != MX_OK) return s;
  return from_hip(mx::launch_dequantize_axis0(codes, scales, y, rows, cols, (int)elem,
                                              reinterpret_cast<hipStream_t>(stream)));
}

mx_status_t mx_fold_scale(uint8_t* scales, int64_t n_scales, int32_t j, mx_stream_t stream) {
  if (!scales) return MX_ERR_NULL;
  if (n_scales < 1) return MX_ERR_SHAPE;
  return from_hip(mx::launch_fold_scale(scales, n_scales, (int)j,
                                        reinterpret_cast<hipStream_t>(stream)));
}

size_t mx_codes_bytes(int64_t rows, int64_t cols, mx_elem_t elem) {
  if (rows < 0 || cols < 0 || !is_elem(elem)) return 0;
  if (cols != 0 && rows > INT64_MAX / cols) return 0;
  const int64_t n = rows * cols;
  return (size_t)(elem == MX_E2M1 ? n / 2 : n);
}

int64_t mx_num_scale_blocks(int64_t rows, int64_t cols, int32_t block_size) {
  if (rows < 0 || cols < 0 || block_size <= 0 || cols % block_size != 0) return 0;
  if (cols != 0 && rows > INT64_MAX / cols) return 0;
  return rows * (cols / block_size);
}

const char* mx_status_string(mx_status_t status) {
  switch (status) {
    case MX_OK: return "ok";
    case MX_ERR_NULL: return "a required pointer is NULL";
    case MX_ERR_SHAPE: return "invalid shape: sizes must be >= 1 and cols/K a multiple of 32";
    case MX_ERR_UNSUPPORTED: return "unsupported element type or block size (E2M1/E4M3, 32)";
    case MX_ERR_ALIGN: return "buffer below the required alignment (16 bytes; 4 for the f32-B product's B and C and the fused product's C)";
    case MX_ERR_HIP: return "HIP runtime error at kernel launch";
  }
  return "unknown status";
}

int32_t mx_abi_version(void) { return LIBMX_ABI_VERSION; }

}  // extern "C"
