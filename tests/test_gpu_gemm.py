"""GPU parity of gemm_f16 against the fp64 GEMM oracle (oracle/gemm_oracle.py).

Bars:
  - integer-valued inputs (|A|, |B| <= 4): every partial sum is an integer below 2^24, so fp32 accumulation
    is exact in any order and C must equal the fp16 rounding (nearest even) of the exact product, bit for
    bit;
  - N(0,1) inputs: |C_gpu - C| <= 2^-11 |C| + 2^-25 + sqrt(K/16 + 16) * 2^-24 * sum_k |A_ik B_kj| per element
    (half an fp16 ulp for the output rounding, plus the probabilistic bound on fp32 accumulation over K/16
    MFMA steps of 16 products each), and the mean error at most 0.35 of the mean fp16 ulp of C (the error
    is the output rounding, not the accumulation).
"""
import math

import numpy as np
import pytest
import torch

from dnn_compiler_pipelining_amd import binding, inputs
from oracle import gemm_oracle as G
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

KN, NK = binding.GEMM_B_KN, binding.GEMM_B_NK


@pytest.fixture(scope="module", autouse=True)
def gpu():
    U.require_gpu()


def mats(M, N, K, layout, seed, dist="normal", lim=0):
    a = inputs.make_matrix(M, K, seed, inputs.MAT_A, dist, lim)
    b = inputs.make_matrix(*((K, N) if layout == KN else (N, K)), seed, inputs.MAT_B, dist, lim)
    return a, b


def run(a, b, layout, M, N, K, guard=4096, waves=0):
    """C on the GPU, from a NaN-filled buffer with a guard region after it that must stay NaN.  `waves` 4 or 8
    picks the workgroup shape (gemm_f16_waves); 0 runs gemm_f16."""
    buf = torch.full((M * N + guard,), float("nan"), dtype=torch.float16, device="cuda")
    if waves:
        st = binding.gemm_f16_waves(a, b, buf, M, N, K, layout, waves, None)
    else:
        st = binding.gemm_f16(a, b, buf, M, N, K, layout, None)
    assert st == binding.ATTN_OK, binding.attn_status_string(st)
    torch.cuda.synchronize()
    assert bool(torch.isnan(buf[M * N:]).all().item()), "write past the end of C"
    return buf[:M * N].view(M, N)


def ulp16(x):
    """Spacing of fp16 numbers at |x| (2^-24 in the subnormal range)."""
    ax = np.maximum(np.abs(x), 2.0 ** -14)
    return 2.0 ** (np.floor(np.log2(ax)) - 10)


def check_normal(c_gpu, ref, absprod, K, tag):
    c = c_gpu.astype(np.float64)
    assert np.isfinite(c).all(), tag
    err = np.abs(c - ref)
    tol = 2.0 ** -11 * np.abs(ref) + 2.0 ** -25 + math.sqrt(K / 16 + 16) * 2.0 ** -24 * absprod
    worst = float((err / tol).max()) if err.size else 0.0
    mean_ratio = float(err.mean() / ulp16(ref).mean()) if err.size else 0.0
    U.say("  %s: max|dC| %.3e, max err/tol %.3f, mean err %.3f ulp" % (tag, float(err.max()), worst, mean_ratio))
    assert worst <= 1.0, tag
    assert mean_ratio <= 0.35, tag


# (M, N, K): one element, exact tiles, ragged M/N/K tails over several tiles, K of one 8-wide chunk; K = 192
# and 128: three and two whole K tiles, where the loads of tile 2 are the only ones issued beside the MFMAs
# (full-tile path) or none are
SHAPES = [(1, 8, 8), (7, 16, 8), (256, 256, 64), (300, 264, 136), (513, 520, 520), (1000, 1024, 1000),
          (64, 8, 4096), (130, 776, 72), (255, 257 - 1, 200), (333, 200, 192), (100, 96, 128)]


@pytest.mark.parametrize("layout", [KN, NK], ids=["kn", "nk"])
@pytest.mark.parametrize("M,N,K", SHAPES, ids=str)
def test_integer_inputs_bit_exact(M, N, K, layout):
    tag = "int M%d N%d K%d layout %d" % (M, N, K, layout)
    U.say(tag)
    a, b = mats(M, N, K, layout, seed=100 + M + N + K, dist="int", lim=4)
    c = run(a.cuda(), b.cuda(), layout, M, N, K)
    want = G.to_f16(G.gemm(a.numpy(), b.numpy(), layout))
    got = c.cpu().numpy()
    bad = np.argwhere(got.view(np.uint16) != want.view(np.uint16))
    assert bad.size == 0, "%s: %d mismatches, first at %s: %r vs %r" % (
        tag, len(bad), tuple(bad[0]), got[tuple(bad[0])], want[tuple(bad[0])])


@pytest.mark.parametrize("layout", [KN, NK], ids=["kn", "nk"])
@pytest.mark.parametrize("M,N,K", SHAPES, ids=str)
def test_normal_inputs(M, N, K, layout):
    tag = "normal M%d N%d K%d layout %d" % (M, N, K, layout)
    U.say(tag)
    a, b = mats(M, N, K, layout, seed=200 + M + N + K)
    c = run(a.cuda(), b.cuda(), layout, M, N, K)
    check_normal(c.cpu().numpy(), G.gemm(a.numpy(), b.numpy(), layout), G.abs_products(a.numpy(), b.numpy(), layout),
                 K, tag)


@pytest.mark.parametrize("name", [w.name for w in inputs.GEMM_WORKLOADS])
def test_full_size_sampled(name):
    """The 8k MatMul workloads as the bench runs them: sampled rows of C against the oracle."""
    w = inputs.GEMM_BY_NAME[name]
    U.say("full size %s" % name)
    a, b = inputs.make_gemm_inputs(w)
    c = run(a.cuda(), b.cuda(), w.b_layout, w.M, w.N, w.K)
    assert bool(torch.isfinite(c).all().item())
    rng = np.random.default_rng(w.seed)
    rows = sorted(set([0, 1, 127, 128, 255, 256, 257, w.M // 2, w.M - 257, w.M - 256, w.M - 1]) |
                  set(int(x) for x in rng.integers(0, w.M, 37)))
    ref = G.gemm_rows(a.numpy(), b.numpy(), w.b_layout, rows)
    absprod = G.abs_products(a.numpy(), b.numpy(), w.b_layout, rows)
    got = c[torch.as_tensor(rows, device=c.device)].cpu().numpy()
    check_normal(got, ref, absprod, w.K, name)


def test_full_size_integer_bit_exact_sampled():
    M = N = K = 8192
    for layout in (KN, NK):
        U.say("full size integer layout %d" % layout)
        a, b = mats(M, N, K, layout, seed=300 + layout, dist="int", lim=2)
        c = run(a.cuda(), b.cuda(), layout, M, N, K)
        rows = [0, 255, 256, 4095, 4096, 8191] + list(range(1000, 1032))
        want = G.to_f16(G.gemm_rows(a.numpy(), b.numpy(), layout, rows))
        got = c[torch.as_tensor(rows, device=c.device)].cpu().numpy()
        assert np.array_equal(got.view(np.uint16), want.view(np.uint16)), layout


def test_layouts_give_the_same_bits():
    """B stored [K,N] and the same B stored [N,K] feed the MFMAs the same values in the same order."""
    M, N, K = 700, 520, 1000
    a, b = mats(M, N, K, KN, seed=401)
    c1 = run(a.cuda(), b.cuda(), KN, M, N, K)
    c2 = run(a.cuda(), b.t().contiguous().cuda(), NK, M, N, K)
    assert torch.equal(c1, c2)


def test_deterministic():
    M, N, K = 1024, 1024, 2048
    a, b = mats(M, N, K, NK, seed=402)
    ad, bd = a.cuda(), b.cuda()
    assert torch.equal(run(ad, bd, NK, M, N, K), run(ad, bd, NK, M, N, K))


def test_k_zero_gives_zeros():
    M, N = 100, 64
    a = torch.empty((M, 0), dtype=torch.float16, device="cuda")
    buf = torch.full((M * N + 64,), float("nan"), dtype=torch.float16, device="cuda")
    st = binding.gemm_f16(a.data_ptr() or 0x1000, 0x2000, buf, M, N, 0, KN, None)
    assert st == binding.ATTN_OK
    torch.cuda.synchronize()
    assert bool((buf[:M * N] == 0).all().item()) and bool(torch.isnan(buf[M * N:]).all().item())


def test_matmul_convenience_matches():
    a, b = mats(300, 264, 136, NK, seed=403)
    ad, bd = a.cuda(), b.cuda()
    c = binding.matmul(ad, bd, NK)
    torch.cuda.synchronize()
    assert torch.equal(c, run(ad, bd, NK, 300, 264, 136))


def test_validation_launches_nothing():
    a, b = mats(64, 64, 64, KN, seed=404)
    c = torch.full((64, 64), float("nan"), dtype=torch.float16, device="cuda")
    st = binding.gemm_f16(a.cuda(), b.cuda(), c, 64, 64, 60, KN, None)  # K not a multiple of 8
    assert st == binding.ATTN_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool(torch.isnan(c).all().item())


@pytest.mark.parametrize("layout", [KN, NK], ids=["kn", "nk"])
@pytest.mark.parametrize("M,N,K", [(300, 264, 136), (513, 520, 520), (1000, 1024, 1000), (64, 8, 4096)], ids=str)
def test_four_wave_workgroups_give_the_same_bits(M, N, K, layout):
    """Workgroups of 4 waves (128 x 128 per wave, 32 x 32 x 16 MFMAs) and of 8 (128 x 64, 16 x 16 x 32 MFMAs)
    feed every output the same products in the same k order, and give the same bits; the 4-wave result also
    meets the oracle bar."""
    a, b = mats(M, N, K, layout, seed=500 + M + K)
    ad, bd = a.cuda(), b.cuda()
    c8 = run(ad, bd, layout, M, N, K, waves=8)
    c4 = run(ad, bd, layout, M, N, K, waves=4)
    assert torch.equal(c8, c4)
    check_normal(c4.cpu().numpy(), G.gemm(a.numpy(), b.numpy(), layout), G.abs_products(a.numpy(), b.numpy(), layout),
                 K, "4 waves M%d N%d K%d layout %d" % (M, N, K, layout))
