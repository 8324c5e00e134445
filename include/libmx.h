/*
 * libmx -- OCP Microscaling (MX) quantize / dequantize / block matmul on
 * AMD Instinct MI355X (gfx950).
 *
 * Formats (all from the "Bit Layout" page, mxfp4community.com, unless noted):
 *   - E2M1 element: 1 sign, 2 exponent (bias 1), 1 mantissa bit; the eight
 *     magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}; no Inf, no NaN
 *     (section "The E2M1 element").
 *   - E4M3 element: f8E4M3FN, 1 sign, 4 exponent (bias 7), 3 mantissa bits,
 *     largest finite magnitude 448, codes 0x7F/0xFF are NaN ("A Dialect Is a
 *     Set of Co-Designed Decisions", section "The type: !mx.tensor").
 *   - E8M0 scale: one unsigned byte per block, value 2^(byte-127); byte 0xFF
 *     is NaN and turns every element of its block into NaN
 *     (section "The E8M0 shared scale").
 *   - A block is 32 contiguous elements along the last (reduction) axis
 *     (section "Block structure and packing"; dialect page, "The block axis").
 *
 * Memory layouts (all row-major, dense, no padding between rows):
 *   - x, y:    float32 [rows, cols]
 *   - codes:   E2M1 -> uint8 [rows, cols/2], element 2j in the low nibble and
 *              element 2j+1 in the high nibble of byte j (section "Block
 *              structure and packing");  E4M3 -> uint8 [rows, cols].
 *   - scales:  uint8 [rows, cols/32]; scale [r, j] covers x[r, 32j .. 32j+31].
 *   - block_matmul takes B transposed, B^T [N, K], so that B's blocks also
 *     run along K, its reduction axis (dialect page, "The block axis": the
 *     block axis must be the reduction axis).  A matrix quantized with
 *     mx_quantize in the [N, K] orientation is a valid B operand.
 *
 * Ownership and asynchrony: every pointer is a device pointer owned by the
 * caller (e.g. from hipMalloc or torch.empty on the GPU).  libmx never
 * allocates, frees or retains a pointer beyond the call.  Work is enqueued on
 * `stream` (NULL = the default stream) and runs asynchronously: synchronize the
 * stream before reading results on the host.  Functions are thread-safe.
 *
 * Errors: arguments are validated before anything is enqueued; on a
 * validation error nothing is launched and nothing is written.  Validation is
 * structural only (null pointers, sizes, divisibility, element type, block
 * size, alignment); data never causes an error: a 0xFF scale decodes to NaN
 * and a block of x holding NaN or Inf quantizes to scale 0xFF with zero
 * codes.  A failed kernel launch returns MX_ERR_HIP, and the outputs are then
 * undefined (one call may enqueue more than one kernel).  Inputs and outputs
 * must not overlap.
 */
#ifndef LIBMX_H
#define LIBMX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LIBMX_ABI_VERSION 3
#define MX_BLOCK_SIZE 32

/* Same object as HIP's hipStream_t (a pointer to the runtime's stream). */
typedef struct ihipStream_t *mx_stream_t;

typedef enum {
  MX_E2M1 = 1, /* MXFP4 element, packed two per byte */
  MX_E4M3 = 2  /* MXFP8 element (f8E4M3FN), one per byte */
} mx_elem_t;

typedef enum {
  MX_OK = 0,
  MX_ERR_NULL = 1,        /* a required pointer is NULL                         */
  MX_ERR_SHAPE = 2,       /* a size < 1, or cols / K not a multiple of 32        */
  MX_ERR_UNSUPPORTED = 3, /* element type not E2M1/E4M3, or block_size != 32     */
  MX_ERR_ALIGN = 4,       /* a pointer below its call's alignment: 16 bytes for   */
                          /* x, y, codes and c; 4 bytes for the f32-B product's  */
                          /* b and c                                             */
  MX_ERR_HIP = 5          /* the HIP runtime reported an error at launch         */
} mx_status_t;

/*
 * mx_quantize -- float32 [rows, cols] -> element codes + E8M0 scales.
 * Follows "Bit Layout", section "Reference encode and decode"; the dialect
 * page, section "The four ops" (quantize_block).  Per block of 32:
 *   amax = max |x_i|;  amax == 0 -> codes 0, scale byte 127;
 *   e = clip(floor(log2 amax) - emax, -127, 127), floor taken exactly
 *   (emax = 2 for E2M1, 8 for E4M3);  scale byte = e + 127;
 *   code_i = index of the grid magnitude nearest to |x_i| / 2^e (ties to the
 *   smaller magnitude, values above the grid saturate to its top)
 *   | sign, where the sign bit is set iff x_i < 0 (so -0.0 gives code 0).
 *   A block holding NaN or Inf gets scale byte 0xFF and zero codes.
 * x: device float32 [rows, cols], 16-byte aligned (read).
 * codes: device, mx_codes_bytes(rows, cols, elem) bytes, 16-byte aligned (written).
 * scales: device, mx_num_scale_blocks(rows, cols, 32) bytes (written).
 * block_size must be 32.
 */
mx_status_t mx_quantize(const float *x, void *codes, uint8_t *scales, int64_t rows,
                        int64_t cols, mx_elem_t elem, int32_t block_size,
                        mx_stream_t stream);

/*
 * mx_dequantize -- element codes + E8M0 scales -> float32 [rows, cols].
 * Follows "Bit Layout", sections "The E8M0 shared scale" and "Reference
 * encode and decode"; the dialect page, section "The four ops"
 * (dequantize_block).  y = (-1)^s * grid[magnitude] * 2^(byte-127), exact;
 * byte 0xFF -> every element of the block is NaN (bits 0x7FC00000), as are
 * E4M3 NaN codes.  Layouts as mx_quantize; y is 16-byte aligned (written).
 */
mx_status_t mx_dequantize(const void *codes, const uint8_t *scales, float *y, int64_t rows,
                          int64_t cols, mx_elem_t elem, int32_t block_size,
                          mx_stream_t stream);

/*
 * mx_block_matmul -- C = [accumulate ? C : 0] + A . B on block-scaled operands.
 * Follows the dialect page, sections "The four ops" (block_matmul, C += A.B),
 * "The block axis" (each block scale is constant along the 32-run of K it
 * multiplies, so it factors out of that partial sum) and "The accumulator
 * operand" (C is both input and output, updated in place).
 *   A:   a_codes [M, K or K/2] + a_scales [M, K/32], element type a_elem.
 *   B^T: b_codes [N, K or K/2] + b_scales [N, K/32], element type b_elem.
 *   C:   device float32 [M, N], 16-byte aligned; read only if accumulate != 0.
 *   C[m,n] = sum_j 2^(sa[m,j]+sb[n,j]-254) * sum_{k in block j} qa[m,k]*qb[n,k]
 * with float32 accumulation; a NaN scale or E4M3 NaN code in row m of A or
 * row n of B^T makes C[m,n] NaN.  Any (a_elem, b_elem) pair of E2M1/E4M3.
 * Accuracy: for E2M1 x E2M1 and the mixed pairs every group of 8 products
 * is summed exactly (an E4M3 operand is split on its exponent into two
 * operands of the matrix instruction), so C differs from the exact sum only
 * by float32 rounding, within 1e-5 * sum_k |a_k b_k| (+ |C_in|), plus up to
 * 2^-146 per block of K where partial sums fall below the normal float32
 * range (there the matrix instruction keeps each scaled contribution only on
 * a grid near the smallest subnormals; measured at most 3.1 * 2^-149 per
 * block).  E4M3 x E4M3
 * uses the instruction's FP8 group sum as it is: each aligned group of 8 K
 * is summed in fixed point with lowest bit 2^(X - 13), X the group's largest
 * exponent sum, smaller products truncated toward zero; that can exceed the
 * bound above where the exponents in a group span more than 7 binades.
 * Scale arrays may have any alignment; the fastest kernel wants both 16-byte
 * aligned with K a multiple of 512, or 4-byte aligned with K a multiple of
 * 128 (other cases take a slower kernel with the same error bound).
 */
mx_status_t mx_block_matmul(const void *a_codes, const uint8_t *a_scales, mx_elem_t a_elem,
                            const void *b_codes, const uint8_t *b_scales, mx_elem_t b_elem,
                            float *c, int64_t M, int64_t N, int64_t K, int32_t block_size,
                            int32_t accumulate, mx_stream_t stream);

/*
 * mx_block_matmul_f32b -- C = [accumulate ? C : 0] + A . B with A block-scaled
 * and B an ordinary float32 matrix.  This is block_matmul as the dialect
 * page's first version defines it (section "The four ops": a block-scaled A
 * of shape MxK, an ordinary f32 B of shape KxN, an accumulator C, C += A.B;
 * section "The accumulator operand": C is updated in place).
 *   A: a_codes [M, K or K/2] + a_scales [M, K/32], element type a_elem;
 *      a_codes 16-byte aligned.
 *   B: device float32 [K, N], row-major, 4-byte aligned (read).
 *   C: device float32 [M, N], 4-byte aligned; read only if accumulate != 0.
 *   C[m,n] = sum_j 2^(sa[m,j]-127) * sum_{k in block j} qa[m,k] * B[k,n]
 * in float32 precision: each product is rounded to float32 or (on the bf16
 * matrix cores, with B split into three exact bf16 parts) exact, partial
 * sums span at most 16 blocks before they are added in float32, and every
 * output lies within 1e-5 * sum_k |a_k b_k| of the exact value (plus up to
 * 2^-146 for each product below the normal float32 range, which is kept only
 * near the subnormal grid); a NaN scale
 * or E4M3 NaN code in row m of A makes row m of C NaN.  A is decoded to
 * float32 as mx_dequantize decodes it, so a code whose value exceeds the
 * float32 range (possible only at scale bytes above 252 for E2M1 or 246 for
 * E4M3, which mx_quantize never writes) is +-Inf there, and the outputs of
 * its row are +-Inf or NaN even where the exact sum is finite.
 * Errors as mx_block_matmul (MX_ERR_ALIGN for a misaligned a_codes, b or c).
 */
mx_status_t mx_block_matmul_f32b(const void *a_codes, const uint8_t *a_scales, mx_elem_t a_elem,
                                 const float *b, float *c, int64_t M, int64_t N, int64_t K,
                                 int32_t block_size, int32_t accumulate, mx_stream_t stream);

/*
 * mx_block_matmul_quantize_a -- C = [accumulate ? C : 0] + Q(A) . B, with A an
 * ordinary float32 matrix quantized inside the product.  The dialect page,
 * section "The four ops": quantize_block is the one lossy step and feeds
 * block_matmul; here the two run as one kernel, so the quantized A is never
 * written to memory.  Q is exactly mx_quantize(A, a_elem) (the same scale
 * bytes and codes, bit for bit), and the product is that of mx_block_matmul
 * on Q(A) and B^T, with the same accuracy per format pair.
 *   A:   device float32 [M, K], row-major, 16-byte aligned (read).
 *   B^T: b_codes [N, K or K/2] (16-byte aligned) + b_scales [N, K/32] (any
 *        alignment), element type b_elem.
 *   C:   device float32 [M, N], 4-byte aligned; read only if accumulate != 0.
 * A block of A holding NaN or Inf gets scale byte 0xFF, so its row of C is
 * NaN.  Each A row is quantized once per 256-column tile of C (N / 256 times
 * in all), which is why the separate mx_quantize + mx_block_matmul stays the
 * faster route for large N.
 * Errors as mx_block_matmul (MX_ERR_ALIGN for a misaligned a, b_codes or c).
 */
mx_status_t mx_block_matmul_quantize_a(const float *a, mx_elem_t a_elem, const void *b_codes,
                                       const uint8_t *b_scales, mx_elem_t b_elem, float *c,
                                       int64_t M, int64_t N, int64_t K, int32_t block_size,
                                       int32_t accumulate, mx_stream_t stream);

/*
 * mx_quantize_axis / mx_dequantize_axis -- the codec with an explicit block
 * axis.  Dialect page, section "The block axis": a block's scale must be
 * constant along the reduction it multiplies, so blocks go on the reduction
 * axis -- the last axis of A [M, K], axis 0 of a K x N matrix B.
 *   axis = 1: blocks x[r, 32j .. 32j+31]; identical to mx_quantize /
 *             mx_dequantize (same layouts, same requirements).
 *   axis = 0: blocks x[32i .. 32i+31, c] of a row-major [rows, cols] float32
 *             matrix; rows must be a multiple of 32.  Storage is block-major,
 *             the layout mx_quantize gives for the transposed matrix:
 *             codes [cols, rows/2] (E2M1, element 32i+2k of column c in the
 *             low nibble of byte 16i+k of codes row c) or [cols, rows] (E4M3),
 *             scales [cols, rows/32].  So mx_quantize_axis(B, axis 0) of a
 *             K x N matrix B yields the B^T operand of mx_block_matmul.
 * Per block, the arithmetic is that of mx_quantize / mx_dequantize.
 * x / y: device float32 [rows, cols], 16-byte aligned; codes 16-byte aligned.
 * Errors: MX_ERR_UNSUPPORTED for axis not 0 or 1, MX_ERR_SHAPE for rows (axis
 * 0) or cols (axis 1) not a multiple of 32; otherwise as mx_quantize.
 */
mx_status_t mx_quantize_axis(const float *x, void *codes, uint8_t *scales, int64_t rows,
                             int64_t cols, int32_t axis, mx_elem_t elem, int32_t block_size,
                             mx_stream_t stream);
mx_status_t mx_dequantize_axis(const void *codes, const uint8_t *scales, float *y, int64_t rows,
                               int64_t cols, int32_t axis, mx_elem_t elem, int32_t block_size,
                               mx_stream_t stream);

/*
 * mx_fold_scale -- in place, turn the scales of a block-scaled tensor X into
 * those of 2^j * X; codes are untouched.  Dialect page, section "The four
 * ops" (fold_scale: a scalar multiply of a block-scaled value folded without
 * touching its elements, exact for powers of two); "Bit Layout", section
 * "The E8M0 shared scale" (byte s is 2^(s-127), 0xFF is NaN).
 * Every scale byte s becomes s + j when s != 0xFF and 0 <= s + j <= 254;
 * otherwise no E8M0 byte represents the product and the byte becomes 0xFF
 * (its block decodes to NaN).  Exact or NaN, never silently rounded.
 * scales: device, n_scales bytes, any alignment (read and written).
 * Errors: MX_ERR_NULL, MX_ERR_SHAPE for n_scales < 1.
 */
mx_status_t mx_fold_scale(uint8_t *scales, int64_t n_scales, int32_t j, mx_stream_t stream);

/* Bytes of the codes of a [rows, cols] tensor: rows*cols/2 (E2M1) or
 * rows*cols (E4M3); 0 for an invalid element type or negative size. */
size_t mx_codes_bytes(int64_t rows, int64_t cols, mx_elem_t elem);

/* Number of E8M0 scales (one per block along the last axis): rows*cols/block_size;
 * dialect page, section "The type: !mx.tensor".  0 for invalid arguments. */
int64_t mx_num_scale_blocks(int64_t rows, int64_t cols, int32_t block_size);

/* Static, NUL-terminated description of a status code. */
const char *mx_status_string(mx_status_t status);

/* LIBMX_ABI_VERSION of the built library. */
int32_t mx_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBMX_H */
