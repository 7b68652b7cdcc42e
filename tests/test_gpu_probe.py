"""GPU test of the measurement aid attn_mfma_ceiling (the sustained dense fp16 MFMA rate of the device on random
operands): it returns a rate between a floor far below any MI355X machine seen and the published dense peak, on the
null stream and on a non-default stream, and rejects bad arguments with nothing launched."""
import ctypes

import pytest
import torch

from dnn_compiler_pipelining_amd import binding
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

PEAK_TFLOPS = 2517.0  # 256 CUs x 2.4 GHz x 4096 dense fp16 FLOP per clock


@pytest.fixture(scope="module", autouse=True)
def gpu():
    U.require_gpu()


def test_rate_is_plausible_on_null_and_side_stream():
    U.say("mfma ceiling, null stream")
    tf = binding.attn_mfma_ceiling(20000)
    assert 400.0 < tf <= PEAK_TFLOPS, tf
    U.say("mfma ceiling, side stream")
    s = torch.cuda.Stream()
    tf2 = binding.attn_mfma_ceiling(20000, s)
    assert 400.0 < tf2 <= PEAK_TFLOPS, tf2


def test_both_instruction_shapes():
    """Both shapes give a plausible rate; the 32 x 32 x 16 one is what attn_mfma_ceiling times (same box, so
    the two agree within a few per cent of clock drift)."""
    U.say("mfma ceiling by shape")
    r32 = binding.attn_mfma_ceiling_shape(32, 20000)
    r16 = binding.attn_mfma_ceiling_shape(16, 20000)
    r = binding.attn_mfma_ceiling(20000)
    U.say("  32x32x16 %.1f, 16x16x32 %.1f, attn_mfma_ceiling %.1f TFLOP/s" % (r32, r16, r))
    for tf in (r32, r16, r):
        assert 400.0 < tf <= PEAK_TFLOPS, (r32, r16, r)
    assert abs(r - r32) <= 0.1 * r32


def test_bad_arguments_launch_nothing():
    lib = binding.load()
    out = ctypes.c_double(-1.0)
    assert lib.attn_mfma_ceiling(0, None, ctypes.byref(out)) == binding.ATTN_ERR_SHAPE
    assert lib.attn_mfma_ceiling(7, None, None) == binding.ATTN_ERR_NULL
    assert lib.attn_mfma_ceiling_shape(24, 7, None, ctypes.byref(out)) == binding.ATTN_ERR_UNSUPPORTED
    assert out.value == -1.0
