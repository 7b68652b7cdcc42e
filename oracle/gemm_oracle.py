"""fp64 oracle of the fp16 GEMM: C = A B (B stored [K, N]) or C = A B^T (B stored [N, K]).

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only tests/, __graft_entry__.smoke()
and the cpu_baseline leg of bench.py may import this module.  It never imports
the GPU package, and the GPU package never imports it.

What it computes.  The GEMM is the "8k MatMul" operator of PipeThreader's
evaluation (page "PipeThreader ... (OSDI 2025)" summary, sections "问题与动机"
and "实验与结果", citing the paper's section 6.4 / Table 4), taken as the plain
matrix product of fp16 operands.  The pages give no epilogue, no scaling and no
output precision.  The plainest reading that fits their fp16 "mma" sTasks (f16
x f16 products contracted into an f32 accumulator: page "AI编译器融合技术 --
5. 并行性与分布式融合", section 5.2.2 "Cooperative Matrix Fusion (MMA)") is
C[i, j] = sum_k A[i, k] B[k, j] over the exact fp16 input values, with an fp16
output rounded to nearest even.

This oracle is that definition in binary64: both operands are widened
exactly (every fp16 value is a binary64 value) and multiplied by numpy's
float64 matmul, a library primitive.  With integer-valued inputs and
|C| < 2^53 the result is exact.  `to_f16` rounds to nearest even (numpy's
float64 -> float16 conversion is correctly rounded).
"""
from __future__ import annotations

import numpy as np

B_KN, B_NK = 0, 1


def _b_as_kn(b: np.ndarray, b_layout: int) -> np.ndarray:
    """B as a [K, N] binary64 matrix, whichever way it is stored."""
    b64 = np.asarray(b, dtype=np.float16).astype(np.float64)
    if b_layout == B_KN:
        return b64
    if b_layout == B_NK:
        return b64.T
    raise ValueError("b_layout must be 0 ([K, N]) or 1 ([N, K])")


def gemm(a: np.ndarray, b: np.ndarray, b_layout: int) -> np.ndarray:
    """C = A B in binary64.  a: fp16 [M, K]; b: fp16 [K, N] (B_KN) or [N, K] (B_NK).  Returns float64 [M, N]."""
    a64 = np.asarray(a, dtype=np.float16).astype(np.float64)
    b64 = _b_as_kn(b, b_layout)
    if a64.ndim != 2 or b64.ndim != 2 or a64.shape[1] != b64.shape[0]:
        raise ValueError("shapes do not chain: A %s, B %s as [K, N]" % (a64.shape, b64.shape))
    return a64 @ b64


def gemm_rows(a: np.ndarray, b: np.ndarray, b_layout: int, rows) -> np.ndarray:
    """Rows `rows` of C = A B in binary64 (float64 [len(rows), N]); for checking sampled rows of a large C."""
    a64 = np.asarray(a, dtype=np.float16)[np.asarray(rows, dtype=np.int64)].astype(np.float64)
    return a64 @ _b_as_kn(b, b_layout)


def abs_products(a: np.ndarray, b: np.ndarray, b_layout: int, rows=None) -> np.ndarray:
    """sum_k |A[i, k]| |B[k, j]| in binary64 (for all rows, or for `rows`): the scale of the rounding error
    of any order of summation."""
    a16 = np.asarray(a, dtype=np.float16)
    if rows is not None:
        a16 = a16[np.asarray(rows, dtype=np.int64)]
    return np.abs(a16.astype(np.float64)) @ np.abs(_b_as_kn(b, b_layout))


def to_f16(c: np.ndarray) -> np.ndarray:
    """Round binary64 values to fp16, to nearest even (overflow gives +-inf)."""
    with np.errstate(over="ignore"):
        return np.asarray(c, dtype=np.float64).astype(np.float16)
