"""attn_fwd_decode_static (split-KV path on the library's own per-GPU workspace) against attn_fwd_decode with a
caller workspace: bit for bit, on two calls in a row (the second smaller, so it runs over what the first left in
the array), plus the fp64 oracle bar, the size limit and invalid arguments."""
import math

import pytest
import torch

from dnn_compiler_pipelining_amd import binding, inputs
from oracle import oracle as oracle_mod
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    U.require_gpu()


def qkv(B, Sq, Sk, Hq, Hkv, D, seed):
    return (inputs.make_tensor(B, Sq, Hq, D, seed, inputs.Q), inputs.make_tensor(B, Sk, Hkv, D, seed, inputs.K),
            inputs.make_tensor(B, Sk, Hkv, D, seed, inputs.V))


def nan_outputs(B, Sq, Hq, D):
    return (torch.full((B, Sq, Hq, D), float("nan"), dtype=torch.float16, device="cuda"),
            torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device="cuda"))


def with_caller_workspace(q, k, v, causal, scale):
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    o, lse = nan_outputs(B, Sq, Hq, D)
    need = binding.attn_decode_workspace_size(B, Sq, Sk, Hq, Hkv, D)
    ws = torch.full(((need + 3) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    st = binding.attn_fwd_decode(q, k, v, o, lse, B, Sq, Sk, Hq, Hkv, D, int(causal), scale, ws, need, None)
    assert st == binding.ATTN_OK, binding.attn_status_string(st)
    torch.cuda.synchronize()
    return o, lse


def with_static_workspace(q, k, v, causal, scale, stream=None):
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    o, lse = nan_outputs(B, Sq, Hq, D)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    st = binding.attn_fwd_decode_static(q, k, v, o, lse, B, Sq, Sk, Hq, Hkv, D, int(causal), scale, stream)
    assert st == binding.ATTN_OK, binding.attn_status_string(st)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    return o, lse


# the larger call fills about half of the array (LLaMA3-70B heads, 16 query rows against 4096 keys); the
# smaller one (8B heads, one query row, a ragged key tail) runs after it over what it left there
CALLS = [(1, 16, 4096, 64, 8, 128, 1, 9101), (2, 1, 1000, 32, 8, 128, 1, 9102)]


def test_two_calls_match_the_caller_workspace_path():
    assert binding.attn_decode_workspace_size(*CALLS[0][:6]) > binding.attn_decode_workspace_size(*CALLS[1][:6])
    stream = torch.cuda.Stream()
    for B, Sq, Sk, Hq, Hkv, D, causal, seed in CALLS:
        tag = "decode_static B%d Sq%d Sk%d Hq%d Hkv%d D%d causal%d" % (B, Sq, Sk, Hq, Hkv, D, causal)
        U.say(tag)
        scale = 1.0 / math.sqrt(D)
        qc, kc, vc = qkv(B, Sq, Sk, Hq, Hkv, D, seed)
        q, k, v = qc.cuda(), kc.cuda(), vc.cuda()
        o_ref, lse_ref = with_caller_workspace(q, k, v, causal, scale)
        o, lse = with_static_workspace(q, k, v, causal, scale, stream)
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), tag + ": O differs from attn_fwd_decode"
        assert torch.equal(lse.view(torch.int32), lse_ref.view(torch.int32)), tag + ": LSE differs"
        O, L = oracle_mod.attn_full(qc.numpy(), kc.numpy(), vc.numpy(), bool(causal), scale)
        U.check(U.stats(o.cpu().numpy(), lse.cpu().numpy(), O, L), tag)


def test_sizes_past_the_array_are_rejected_untouched():
    B, Sq, Sk, Hq, Hkv, D = 1, 128, 8192, 64, 8, 256
    assert binding.attn_decode_workspace_size(B, Sq, Sk, Hq, Hkv, D) > binding.ATTN_STATIC_WORKSPACE_BYTES
    U.say("decode_static too large B%d Sq%d Sk%d Hq%d Hkv%d D%d" % (B, Sq, Sk, Hq, Hkv, D))
    q = torch.zeros((B, Sq, Hq, D), dtype=torch.float16, device="cuda")
    k = torch.zeros((B, Sk, Hkv, D), dtype=torch.float16, device="cuda")
    v = torch.zeros_like(k)
    o, lse = nan_outputs(B, Sq, Hq, D)
    st = binding.attn_fwd_decode_static(q, k, v, o, lse, B, Sq, Sk, Hq, Hkv, D, 1, 0.0625, None)
    assert st == binding.ATTN_ERR_TOO_LARGE
    torch.cuda.synchronize()
    assert torch.isnan(o).all() and torch.isnan(lse).all()


def test_invalid_arguments_keep_the_decode_codes():
    q = torch.zeros((1, 1, 6, 128), dtype=torch.float16, device="cuda")
    k = torch.zeros((1, 64, 4, 128), dtype=torch.float16, device="cuda")
    o, lse = nan_outputs(1, 1, 6, 128)
    assert binding.attn_fwd_decode_static(q, k, k, o, lse, 1, 1, 64, 6, 4, 128, 1, 0.1, None) == \
        binding.ATTN_ERR_SHAPE  # Hq % Hkv != 0
    assert binding.attn_fwd_decode_static(None, k, k, o, lse, 1, 1, 64, 4, 4, 128, 1, 0.1, None) == \
        binding.ATTN_ERR_NULL
    torch.cuda.synchronize()
    assert torch.isnan(o).all()
