"""CPU tests: the fp64 oracle against its pins (no GPU)."""
import numpy as np
import pytest

from oracle import oracle as oracle_mod
from tests import oracle_pins as P


@pytest.fixture(scope="module")
def orc():
    return oracle_mod.default()


def test_half_to_double_every_bit_pattern(orc):
    """The oracle's own fp16 decoder against numpy's conversion, all 65536 patterns."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    want = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.half_to_double(int(b)) for b in bits])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(orc, pin):
    pin(orc)


def test_rows_matches_full(orc):
    """The per-row entry point (used for sampled checks at full size) equals the whole-tensor one."""
    rng = np.random.default_rng(3)
    q, k, v = P.rand_qkv(rng, 2, 37, 8, 2, 16)
    O, L = orc.full(q, k, v, True, 0.2)
    heads = [0, 7, 3, 3, 5]
    rows = [36, 0, 17, 18, 1]
    o, lse = orc.rows(q[1], k[1], v[1], heads, rows, True, 0.2, nthreads=3)
    for n, (h, i) in enumerate(zip(heads, rows)):
        assert np.array_equal(o[n], O[1, i, h])
        assert lse[n] == L[1, h, i]


def test_thread_count_does_not_change_results(orc):
    rng = np.random.default_rng(4)
    q, k, v = P.rand_qkv(rng, 1, 50, 4, 1, 32)
    a = orc.full(q, k, v, True, 0.3, nthreads=1)
    b = orc.full(q, k, v, True, 0.3, nthreads=7)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_rejects_bad_arguments(orc):
    rng = np.random.default_rng(5)
    q, k, v = P.rand_qkv(rng, 1, 4, 3, 2, 8)  # Hq % Hkv != 0
    with pytest.raises(RuntimeError):
        orc.rows(q[0], k[0], v[0], [0], [0], True, 0.1)
    q, k, v = P.rand_qkv(rng, 1, 4, 2, 1, 8)
    with pytest.raises(RuntimeError):
        orc.rows(q[0], k[0], v[0], [2], [0], True, 0.1)  # head out of range
    with pytest.raises(RuntimeError):
        orc.rows(q[0], k[0], v[0], [0], [4], True, 0.1)  # row out of range


def test_rejects_causal_with_more_queries_than_keys(orc):
    """Bottom-right causal alignment needs Sq <= Sk (every row keeps a key); non-causal allows any."""
    rng = np.random.default_rng(4)
    q = rng.standard_normal((5, 2, 8)).astype(np.float16)
    k = rng.standard_normal((3, 1, 8)).astype(np.float16)
    with pytest.raises(RuntimeError):
        orc.rows(q, k, k, [0], [0], True, 0.5)
    o, lse = orc.rows(q, k, k, [0, 1], [4, 0], False, 0.5)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
