/*
 * gemm.h -- C ABI of libattn's fp16 GEMM for AMD Instinct MI355X (gfx950).
 *
 * The operation.  PipeThreader's evaluation compiles an 8k MatMul and quotes
 * the tensor-core utilisation that a hardware-scheduled MatMul reaches (page
 * "PipeThreader: Software-Defined Pipelining for Efficient DNN Execution (OSDI
 * 2025)" summary, sections "问题与动机" and "实验与结果", citing the paper's
 * section 6.4 / Table 4).  Its mma sTasks contract fp16 operands into an fp32
 * accumulator (page "AI编译器融合技术 -- 5. 并行性与分布式融合", section 5.2.2
 * "Cooperative Matrix Fusion (MMA)").  gemm_f16 computes
 *
 *   C[i][j] = sum_{k < K} A[i][k] * B[k][j]        (b_layout = GEMM_B_KN)
 *   C[i][j] = sum_{k < K} A[i][k] * B[j][k]        (b_layout = GEMM_B_NK)
 *
 * with fp16 inputs, products and sums in fp32 (the order of the sums is the
 * library's), and C rounded to fp16, to nearest even.  K = 0 gives C = 0.
 *
 * Tensors (device memory, owned and allocated by the caller, row-major and
 * contiguous):
 *   a  fp16 [M][K]
 *   b  fp16 [K][N] (GEMM_B_KN: C = A B)  or  [N][K] (GEMM_B_NK: C = A B^T,
 *      the layout of a linear layer's weight)
 *   c  fp16 [M][N] (written; must not overlap a or b)
 * Every pointer must be 16-byte aligned.
 *
 * Scalars: 0 <= M, N <= 2^24 and 0 <= K <= 2^22, with at most 2^31 - 1
 * output tiles of 256 x 256; K and N must be multiples of 8, so that every
 * row starts 16-byte aligned (ATTN_ERR_UNSUPPORTED otherwise).  M = 0 or
 * N = 0 launches nothing and returns ATTN_OK; the pointers may then be NULL.
 *
 * Execution: the call validates its arguments, then enqueues one kernel on
 * the given HIP stream (a hipStream_t; NULL means the null stream) and
 * returns without waiting.  The library allocates no memory, keeps no state
 * between calls, is thread-safe, and gives bitwise identical results run to
 * run.
 *
 * Errors: the status codes of attn.h.  On invalid arguments nothing is
 * launched: ATTN_ERR_NULL (a, b or c NULL with M, N > 0), ATTN_ERR_SHAPE (a
 * size out of range, b_layout not 0 or 1, too many output tiles),
 * ATTN_ERR_UNSUPPORTED (K or N not a multiple of 8), ATTN_ERR_ALIGN,
 * ATTN_ERR_OVERLAP (c overlaps a or b); ATTN_ERR_HIP if the launch fails.
 * Checks run in that order.
 */
#ifndef LIBATTN_GEMM_H
#define LIBATTN_GEMM_H

#include "attn.h"

#ifdef __cplusplus
extern "C" {
#endif

enum { GEMM_B_KN = 0, GEMM_B_NK = 1 };

/* C = A B or A B^T (see above), enqueued on `stream`.  Returns ATTN_OK or an ATTN_ERR_* code. */
int gemm_f16(const void* a, const void* b, void* c, int M, int N, int K, int b_layout, void* stream);

/* gemm_f16 with an explicit workgroup shape, for tuning and cross-checks: `waves` 8 (eight waves of
 * 128 x 64 outputs each on 16 x 16 x 32 MFMAs, the default), 4 (four waves of 128 x 128 on 32 x 32 x 16
 * MFMAs, accumulators in AGPRs) or 0 (the default).  Both shapes give bitwise identical results (the
 * products of each output meet its fp32 accumulator in the same order and groups on either MFMA).  Any other value returns ATTN_ERR_UNSUPPORTED
 * after the argument checks above. */
int gemm_f16_waves(const void* a, const void* b, void* c, int M, int N, int K, int b_layout, int waves,
                   void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBATTN_GEMM_H */
