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


def test_bad_arguments_launch_nothing():
    lib = binding.load()
    out = ctypes.c_double(-1.0)
    assert lib.attn_mfma_ceiling(0, None, ctypes.byref(out)) == binding.ATTN_ERR_SHAPE
    assert lib.attn_mfma_ceiling(7, None, None) == binding.ATTN_ERR_NULL
    assert out.value == -1.0
