/*
 * qk.h - C ABI of libqk: ggml block-quantized dequantize, GEMV and GEMM on
 * AMD gfx950 (MI355X).
 *
 * Block formats (32 weights per block, little-endian binary16 fields, blocks
 * packed back to back, a matrix stored row after row with k/32 blocks per row
 * and no padding):
 *   QK_Q4_0  d[2] qs[16]       18 bytes  w = d*q + (-8*d),  q = nibble 0..15
 *   QK_Q4_1  d[2] m[2] qs[16]  20 bytes  w = d*q + m
 *   QK_Q8_0  d[2] qs[32]       34 bytes  w = d*q,           q = int8
 *   QK_Q5_0  d[2] qh[4] qs[16] 22 bytes  w = (q - 16) * d,  q = 0..31
 *   QK_Q5_1  d[2] m[2] qh[4] qs[16]  24 bytes  w = d*q + m, q = 0..31
 * For Q4_x, quant byte j holds element j in its low nibble and element j+16 in
 * its high nibble.  Source: "llama_cpp 0.12.1 -> 0.12.2" diff of ggml-cuda.cu
 * (diffend, page 4), hunks adding dequantize_block_q4_0, dequantize_block_q4_1
 * and dequantize_block_q8_0_f16; the row launchers dequantize_row_q4_*_cuda
 * give the 32-weight block (nb32 = k/32).
 * Q5_x: the same diff names these formats only in ggml_get_to_fp16_cuda /
 * ggml_get_to_fp32_cuda (dequantize_block_cuda with dequantize_q5_0 / _q5_1);
 * their layout is not printed there and follows ggml's block format: the low
 * four bits of each code as in Q4_x, bit 4 of code t in bit t of qh (a
 * little-endian 32-bit word).  Q5_0's (q - 16) * d makes q = 16 with d < 0
 * a -0.0 (Q4_0's form gives +0.0).
 *
 * Matrix layout follows ggml (ne0 is the contiguous dimension):
 *   W  m rows of k weights (row-major blocks as above);
 *   X  n activation columns of length k, column j starting at element j*ldx;
 *   Y  n output columns of length m, column j starting at element j*ldy.
 *
 * Conventions shared by every call:
 *   - Pointers are device pointers (or host-registered/managed memory the GPU
 *     can read) owned by the caller; they are borrowed until the enqueued work
 *     completes.  The library allocates, frees and synchronizes nothing and
 *     keeps no state, so calls are re-entrant.
 *   - `stream` is a hipStream_t passed as void*; NULL is the null stream.  Work
 *     is enqueued on it and the call returns without waiting.
 *   - The return value is QK_OK or an error code.  When validation fails,
 *     nothing is enqueued.  The library never aborts or prints.
 *   - m == 0, rows == 0 or n == 0 is a no-op returning QK_OK.
 *   - k must be a non-negative multiple of 32 (QK_ERR_INVALID_ARG otherwise).
 *   - Output ranges must not overlap input ranges (QK_ERR_INVALID_ARG).
 */
#ifndef QK_H
#define QK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Block formats (this library's own numbering). */
enum qk_format {
    QK_Q4_0 = 1,
    QK_Q4_1 = 2,
    QK_Q8_0 = 3,
    QK_Q5_0 = 4,
    QK_Q5_1 = 5
};

/* Output element types of qk_dequantize. */
enum qk_dtype {
    QK_F32 = 0,
    QK_F16 = 1
};

/* Status codes. */
enum qk_status {
    QK_OK = 0,
    QK_ERR_INVALID_ARG = 1,   /* null pointer, bad size, k % 32 != 0, n out of
                                 range, ld too small, overlapping in/out */
    QK_ERR_UNSUPPORTED = 2,   /* unknown format or output dtype */
    QK_ERR_ALIGNMENT = 3,     /* w not 2-byte aligned, or x / y / out not
                                 aligned to their element size */
    QK_ERR_LAUNCH = 4         /* the HIP runtime refused the kernel launch */
};

/* Bytes per 32-weight block: 18, 20, 34, 22 or 24; 0 for an unknown format. */
size_t qk_block_bytes(int fmt);

/* Bytes of one row of k weights (k a multiple of 32); 0 on a bad argument. */
size_t qk_row_bytes(int fmt, int64_t k);

/* Static, human-readable name of a status code (never NULL). */
const char *qk_status_string(int status);

/* Library version as an integer (major*10000 + minor*100 + patch). */
int qk_version(void);

/*
 * qk_dequantize - convert a rows x k quantized matrix to fp32 or fp16.
 *
 *   out[r*k + c] = W[r, c]   for r < rows, c < k.
 *
 * fp32: the value is computed in fp32 in the order shown in the format table
 * (multiply, then add; no fused multiply-add), which is exact for Q4_0, Q8_0
 * and Q5_0 and one round-to-nearest-even for Q4_1 and Q5_1.  Q4_0 with q = 8
 * gives +0.0; Q5_0 with q = 16 gives a zero with the sign of d.
 * fp16: one round-to-nearest-even of that fp32 value (overflow to +-inf,
 * subnormals kept).
 * Source: dequantize_block_q4_0 / _q4_1 / _q8_0_f16 hunks and the
 * ggml_get_to_fp16_cuda / ggml_get_to_fp32_cuda dispatch in the same diff.
 *
 *   fmt        QK_Q4_0, QK_Q4_1, QK_Q8_0, QK_Q5_0 or QK_Q5_1
 *   w          rows*k/32 blocks; 2-byte aligned
 *   rows, k    rows >= 0, k >= 0, k % 32 == 0
 *   out_dtype  QK_F32 or QK_F16
 *   out        rows*k elements of out_dtype, aligned to the element size
 *   stream     hipStream_t or NULL
 */
int qk_dequantize(int fmt, const void *w, int64_t rows, int64_t k,
                  int out_dtype, void *out, void *stream);

/*
 * qk_mul_mat_vec - fused quantized GEMV for decode: dequantize in registers
 * and multiply by 1..8 fp32 activation vectors, accumulating in fp32.
 *
 *   y[j*ldy + i] = sum_c W[i, c] * x[j*ldx + c]   for i < m, j < n   (overwrite)
 *
 * Each product uses the exact fp32 weight value, so the result is within a
 * few fp32 roundings per term of the exact sum: |y - exact| is a small
 * multiple of 2^-24 * sum_c |W[i,c] x[j*ldx+c]|.  With 4..8 columns, weights
 * 4-byte aligned with an even block count and k <= 4096, the multiply-adds
 * run on the matrix cores (fp32 MFMA, each a fused multiply-add with one
 * rounding, like the vector ALU's), in a different order than the vector-ALU
 * kernel the other cases use.
 * Source: dequantize_mul_mat_vec (the "dmmv" tuning block) and the
 * ggml_cuda_op_mul_mat row-range x column-count driver in the same diff,
 * which use it when the right operand is a vector.
 *
 *   w          m rows of k/32 blocks; 2-byte aligned
 *   m, k       m >= 0, k >= 0, k % 32 == 0
 *   x          fp32, 4-byte aligned; n columns, stride ldx >= k
 *   n          0..8 (0 is a no-op; above 8: QK_ERR_INVALID_ARG)
 *   y          fp32, 4-byte aligned; n columns, stride ldy >= m
 */
int qk_mul_mat_vec(int fmt, const void *w, int64_t m, int64_t k,
                   const float *x, int64_t n, int64_t ldx,
                   float *y, int64_t ldy, void *stream);

/*
 * qk_mul_mat_vec_x8 - quantized GEMV with 8-bit activations and integer dot
 * products: as qk_mul_mat_vec, but every 32-element block of each activation
 * column is first quantized (inside the kernel, no scratch memory) to codes
 * q = round-half-even(x / d) with a power-of-two scale d = 2^e, e the
 * smallest integer >= -126 with 127 * 2^e >= max|x| over the block (d = 0 for
 * an all-zero block; d = NaN for a block holding an infinite or NaN value,
 * so every output that uses such a block is NaN), and the products use
 * x^ = d * q:
 *
 *   y[j*ldy + i] = sum_c W[i, c] * x^[j][c]      for i < m, j < n   (overwrite)
 *
 * Per block the weight and activation codes meet in exact 4-way int8 dot
 * products; the result is scaled by d_w * d in fp32 (and Q4_1 adds
 * m_w * d * sum q), so |y - sum_c W x^| is a few fp32 roundings of those
 * per-block terms.  Against the fp32 activations the quantization adds at
 * most sum_c |W[i, c]| * d / 2.
 * Source: the integer-dot GEMV (mul_mat_vec_q, fed by a q8_1 activation
 * quantization) that the "llama_cpp 0.12.1 -> 0.12.2" ggml-cuda.cu diff names
 * in ggml_cuda_mul_mat's kernel choice; its activation format is not on the
 * page, and the power-of-two block scale is this library's.
 *
 * Arguments, layouts and errors as qk_mul_mat_vec (n = 1..8).
 */
int qk_mul_mat_vec_x8(int fmt, const void *w, int64_t m, int64_t k,
                      const float *x, int64_t n, int64_t ldx,
                      float *y, int64_t ldy, void *stream);

/* One problem of a grouped GEMV: y = W x (layout as in qk_mul_mat_vec). */
typedef struct qk_mat_vec_item {
    const void *w;      /* m rows of k/32 blocks, 2-byte aligned */
    int64_t m;          /* rows, m >= 0 (0: skipped) */
    int64_t k;          /* weights per row, k >= 0, k % 32 == 0 */
    const float *x;     /* n fp32 columns of length k, stride ldx >= k */
    int64_t ldx;
    float *y;           /* n fp32 columns of length m, stride ldy >= m */
    int64_t ldy;
} qk_mat_vec_item;

/* Largest `count` qk_mul_mat_vec_batched accepts. */
#define QK_MAX_BATCH 16

/*
 * qk_mul_mat_vec_batched - several independent GEMVs of one format and one
 * column count n in a single launch (for example the q/k/v/o, gate/up and down
 * projections of one decode step, or a set of expert matrices); one launch
 * amortizes the fixed launch cost over all items' weights.  Each item is
 * computed exactly as qk_mul_mat_vec would compute it, bit for bit, except
 * where a single call of 4..8 columns would take the matrix-core kernel: a
 * grouped launch computes every item on the vector ALU, and the two agree
 * within the error bound.  (A one-item call is a single call.)
 * Source: as qk_mul_mat_vec (dequantize_mul_mat_vec under ggml_cuda_op_mul_mat,
 * "llama_cpp 0.12.1 -> 0.12.2" ggml-cuda.cu diff), applied per item.
 *
 *   items      host array of `count` problems (read during the call only)
 *   count      0..QK_MAX_BATCH (0 is a no-op)
 *   n          1..8 columns for every item (0 is a no-op)
 * Errors as qk_mul_mat_vec for each item; additionally QK_ERR_INVALID_ARG for
 * count out of range, items == NULL with count > 0, or an output overlapping
 * any input or any other item's output.
 */
int qk_mul_mat_vec_batched(int fmt, const qk_mat_vec_item *items, int count, int64_t n,
                           void *stream);

/*
 * qk_mul_mat_vec_id - expert-indexed GEMV for mixture-of-experts decode: for
 * every token t and slot s, the GEMV of the expert matrix that ids selects,
 * with the expert id read on the device (no host synchronisation).
 *
 *   e = ids[t*ld_ids + s]
 *   y[t*y_tok + s*y_slot + i] = sum_c W_e[i, c] * x[t*x_tok + s*x_slot + c]
 *        for i < m, s < n_used, t < n_tokens                          (overwrite)
 *   W_e = m rows of k/32 blocks starting at byte e*expert_stride of w
 *
 * Each (t, s) is computed exactly as qk_mul_mat_vec computes one column.  An
 * id outside [0, n_experts) selects nothing: its m outputs are set to NaN and
 * no weight outside the stack is read.
 * Source: ggml_cuda_mul_mat_id, named by a ggml-cuda.cu hunk of the
 * "ggml: backend-agnostic tensor parallelism" compare (whose commit list
 * mentions a Q4_0 expert model with intermediate dimension 768); its
 * definition is not printed there, and this follows ggml's mul_mat_id: one
 * product per (token, selected expert).
 *
 *   w              stack of n_experts matrices, 2-byte aligned
 *   n_experts      >= 1
 *   expert_stride  bytes between experts, even, >= one matrix (ignored if
 *                  n_experts == 1)
 *   m, k           m >= 0, k >= 0, k % 32 == 0
 *   ids            device int32, 4-byte aligned; token t's ids at t*ld_ids
 *   ld_ids         >= n_used (ignored if n_tokens == 1)
 *   n_used         slots per token, >= 0 (0 is a no-op)
 *   n_tokens       >= 0 (0 is a no-op)
 *   x              fp32, 4-byte aligned; x_slot = 0 gives every slot of a
 *                  token the same vector; strides >= 0, in elements
 *   y              fp32, 4-byte aligned; the n_used*n_tokens outputs must not
 *                  overlap: (y_slot >= m and y_tok >= (n_used-1)*y_slot + m)
 *                  or (y_tok >= m and y_slot >= (n_tokens-1)*y_tok + m)
 * Errors: QK_ERR_INVALID_ARG for the conditions above, n_used * n_tokens *
 * ceil(m/8) above INT32_MAX, a null pointer, or y overlapping w, ids or x;
 * QK_ERR_ALIGNMENT as listed; nothing is enqueued on an error.
 */
int qk_mul_mat_vec_id(int fmt, const void *w, int64_t n_experts, int64_t expert_stride,
                      int64_t m, int64_t k, const int32_t *ids, int64_t ld_ids,
                      int64_t n_used, int64_t n_tokens,
                      const float *x, int64_t x_slot, int64_t x_tok,
                      float *y, int64_t y_slot, int64_t y_tok, void *stream);

/*
 * qk_mul_mat - batched GEMM: weights dequantized to fp16 tiles in LDS and
 * multiplied by fp16 activations on the matrix cores, accumulating in fp32.
 *
 *   y[j*ldy + i] = sum_c f16(W[i, c]) * x[j*ldx + c]   for i < m, j < n
 *
 * f16(W) is the qk_dequantize fp16 value (one RNE of the fp32 weight).
 * Every format.
 * Source: the dequantize-to-fp16 then GEMM path (ggml_get_to_fp16_cuda feeding
 * the BLAS mul_mat) and ggml_cuda_mul_mat's choice of a batched kernel when
 * the right operand has more than one column, in the same diff.
 *
 *   x          binary16, 2-byte aligned; n columns, stride ldx >= k
 *   n          n >= 0
 *   y          fp32, 4-byte aligned; n columns, stride ldy >= m
 */
int qk_mul_mat(int fmt, const void *w, int64_t m, int64_t k,
               const void *x_f16, int64_t n, int64_t ldx,
               float *y, int64_t ldy, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QK_H */
