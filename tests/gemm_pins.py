"""Pins of the fp64 GEMM oracle (oracle/gemm_oracle.py) to facts outside it.

Each pin takes the oracle module (or a planted-mistake copy of it) and raises
AssertionError when the oracle disagrees with:
  - hand-worked products and fp16 roundings (tests/golden/gemm_handworked.json);
  - brute force: a pure-Python triple loop in exact rational arithmetic;
  - closed forms: identity and all-ones operands, outer products;
  - invariants: the two B layouts agree, (A B)^T = B^T A^T, sampled rows equal full rows;
  - special cases: K = 0 gives zeros, integer inputs give exact integers.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "gemm_handworked.json")
B_KN, B_NK = 0, 1


def _f16(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16)


def _rng_f16(rng, shape, scale=1.0):
    return (rng.standard_normal(shape) * scale).astype(np.float16)


def _exact_product(a16, bkn16):
    """C = A B with Fractions: a pure-Python triple loop, no library arithmetic."""
    M, K = a16.shape
    N = bkn16.shape[1]
    A = [[Fraction(float(a16[i, k])) for k in range(K)] for i in range(M)]
    B = [[Fraction(float(bkn16[k, j])) for j in range(N)] for k in range(K)]
    C = [[Fraction(0)] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            s = Fraction(0)
            for k in range(K):
                s += A[i][k] * B[k][j]
            C[i][j] = s
    return C


def pin_handworked(orc):
    with open(GOLDEN) as f:
        g = json.load(f)
    for case in g["products"]:
        a = _f16(case["a"])
        bkn = _f16(case["b_kn"])
        want = np.asarray(case["expected"], dtype=np.float64)
        assert np.array_equal(orc.gemm(a, bkn, B_KN), want), case["name"]
        assert np.array_equal(orc.gemm(a, np.ascontiguousarray(bkn.T), B_NK), want), case["name"] + " (B stored [N,K])"
    for r in g["to_f16"]:
        got = float(orc.to_f16(np.array([r["x"]], dtype=np.float64))[0])
        want = float("inf") if r["expected"] == "inf" else float(r["expected"])
        assert got == want or (np.isinf(got) and np.isinf(want)), (r, got)
        assert float(np.float16(want)) == want or np.isinf(want)


def pin_brute_force(orc, seed=31):
    rng = np.random.default_rng(seed)
    for M, N, K in [(1, 1, 1), (3, 5, 7), (4, 2, 9), (5, 6, 3), (2, 7, 16)]:
        a = _rng_f16(rng, (M, K))
        bkn = _rng_f16(rng, (K, N))
        ref = _exact_product(a, bkn)
        for layout, b in ((B_KN, bkn), (B_NK, np.ascontiguousarray(bkn.T))):
            c = orc.gemm(a, b, layout)
            assert c.shape == (M, N), (c.shape, M, N)
            for i in range(M):
                for j in range(N):
                    err = abs(Fraction(float(c[i, j])) - ref[i][j])
                    assert err <= Fraction(1, 1 << 40) * (1 + abs(ref[i][j])), (M, N, K, layout, i, j)
        rows = [M - 1, 0]
        cr = orc.gemm_rows(a, bkn, B_KN, rows)
        for n, i in enumerate(rows):
            for j in range(N):
                assert abs(Fraction(float(cr[n, j])) - ref[i][j]) <= Fraction(1, 1 << 40) * (1 + abs(ref[i][j]))
        ab = orc.abs_products(a, bkn, B_KN)
        for i in range(M):
            for j in range(N):
                s = sum(abs(float(a[i, k])) * abs(float(bkn[k, j])) for k in range(K))
                assert abs(ab[i, j] - s) <= 1e-12 * (1 + s), (i, j)


def pin_identity_and_ones(orc, seed=32):
    rng = np.random.default_rng(seed)
    K, N = 12, 5
    bkn = _rng_f16(rng, (K, N))
    eye = np.eye(K, dtype=np.float16)
    assert np.array_equal(orc.gemm(eye, bkn, B_KN), bkn.astype(np.float64))
    bnk = np.ascontiguousarray(bkn.T)
    assert np.array_equal(orc.gemm(eye, bnk, B_NK), bkn.astype(np.float64))
    ones = np.ones((3, K), dtype=np.float16)
    c = orc.gemm(ones, bkn, B_KN)
    for j in range(N):
        col = sum(Fraction(float(bkn[k, j])) for k in range(K))
        for i in range(3):
            assert abs(Fraction(float(c[i, j])) - col) <= Fraction(1, 1 << 40), (i, j)


def pin_outer_product(orc):
    u = _f16([[1], [-2], [3], [0.5]])
    v = _f16([[2, -1, 0.25]])
    c = orc.gemm(u, v, B_KN)
    for i in range(4):
        for j in range(3):
            assert c[i, j] == float(u[i, 0]) * float(v[0, j])


def pin_layouts_and_transpose(orc, seed=33):
    rng = np.random.default_rng(seed)
    a = rng.integers(-3, 4, (6, 10)).astype(np.float16)
    bkn = rng.integers(-3, 4, (10, 4)).astype(np.float16)
    c1 = orc.gemm(a, bkn, B_KN)
    c2 = orc.gemm(a, np.ascontiguousarray(bkn.T), B_NK)
    assert np.array_equal(c1, c2)
    ct = orc.gemm(np.ascontiguousarray(bkn.T), np.ascontiguousarray(a.T), B_KN)
    assert np.array_equal(c1.T, ct)


def pin_integer_exact(orc, seed=34):
    """Integer operands: the product is an exact integer, compared with Python integer sums."""
    rng = np.random.default_rng(seed)
    M, N, K = 3, 4, 257
    ai = rng.integers(-4, 5, (M, K))
    bi = rng.integers(-4, 5, (K, N))
    c = orc.gemm(ai.astype(np.float16), bi.astype(np.float16), B_KN)
    for i in range(M):
        for j in range(N):
            assert c[i, j] == sum(int(ai[i, k]) * int(bi[k, j]) for k in range(K)), (i, j)


def pin_empty(orc):
    a = np.zeros((3, 0), dtype=np.float16)
    b = np.zeros((0, 5), dtype=np.float16)
    c = orc.gemm(a, b, B_KN)
    assert c.shape == (3, 5) and not c.any()
    c = orc.gemm(a, np.zeros((5, 0), dtype=np.float16), B_NK)
    assert c.shape == (3, 5) and not c.any()
    assert orc.gemm(np.zeros((0, 4), dtype=np.float16), np.zeros((4, 2), dtype=np.float16), B_KN).shape == (0, 2)


ALL_PINS = [pin_handworked, pin_brute_force, pin_identity_and_ones, pin_outer_product, pin_layouts_and_transpose,
            pin_integer_exact, pin_empty]
