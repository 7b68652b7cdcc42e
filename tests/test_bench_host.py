"""Host logic of bench.py (no GPU): the launch counts of the timed region and the kernel source fingerprint."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_counts_given_on_the_command_line_are_used_as_given():
    assert bench.launch_counts(1.0, 7, 2, False) == (7, 2)
    assert bench.launch_counts(88.0, 20, 3, False) == (20, 3)
    assert bench.launch_counts(0.01, 1, 0, False) == (1, 0)


def test_default_counts_give_short_workloads_a_quarter_second():
    # the bench workload (~88 ms per launch): the plain defaults
    assert bench.launch_counts(88.0, None, None, False) == (20, 3)
    # a ~1.4 ms GEMM: at least 0.25 s of warmup and of timed launches
    k, w = bench.launch_counts(1.37, None, None, False)
    assert k * 1.37 >= 250.0 and w * 1.37 >= 250.0 and k == w
    # one of the two given: that one exact, the other by the rule
    assert bench.launch_counts(1.37, 5, None, False) == (5, w)
    # launch-bound shapes stop at 5000 launches
    assert bench.launch_counts(0.001, None, None, False) == (5000, 5000)


def test_all_takes_at_least_the_given_counts():
    k, w = bench.launch_counts(1.37, None, None, True)
    assert bench.launch_counts(1.37, 3, 1, True) == (k, w)
    assert bench.launch_counts(88.0, 50, 10, True) == (50, 10)


def test_fingerprint_separates_attention_and_gemm_sources():
    fa = bench.kernel_fingerprint("llama3-70b_b64_s8192")
    fg = bench.kernel_fingerprint("gemm_8k_nt")
    assert len(fa) == 16 and len(fg) == 16 and fa != fg
    assert bench.kernel_fingerprint("llama3-8b_b64_s2048") == fa


def test_variant_shape_pairs_match_a_brute_force_mask():
    """The FLOP count of the variant lines: (query, key) pairs under the bottom-right causal mask (query
    row i sees keys 0..i + Sk - Sq), counted on an explicit mask, and Sq * Sk without it."""
    import numpy as np

    from dnn_compiler_pipelining_amd import inputs

    for Sq, Sk in ((1, 1), (1, 64), (7, 200), (100, 100), (129, 700), (300, 301)):
        i = np.arange(Sq)[:, None]
        j = np.arange(Sk)[None, :]
        mask = j <= i + (Sk - Sq)
        w = inputs.VariantShape("t", 2, Sq, Sk, 8, 2, 128, True, 0)
        assert w.pairs == int(mask.sum()), (Sq, Sk)
        assert inputs.VariantShape("t", 2, Sq, Sk, 8, 2, 128, False, 0).pairs == Sq * Sk
        assert w.flops == 4.0 * 128 * 2 * 8 * int(mask.sum())
    assert {w.D for w in inputs.VARIANT_SHAPES} == {64, 128, 256}
    assert any(not w.causal for w in inputs.VARIANT_SHAPES) and any(w.Sq < w.Sk for w in inputs.VARIANT_SHAPES)
    assert [inputs.scale_for(D) for D in (64, 128, 256)] == [0.125, inputs.SCALE_D128, 0.0625]
