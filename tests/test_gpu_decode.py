"""GPU parity of attn_fwd_decode (split-KV path) against the fp64 oracle, same bar as tests/test_gpu_parity.py.

The workspace is filled with NaN before each call, so a partial that is read before it is written fails."""
import math

import numpy as np
import pytest
import torch

from dnn_compiler_pipelining_amd import binding, inputs
from oracle import oracle as oracle_mod
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    U.require_gpu()


def cpu_qkv(B, Sq, Sk, Hq, Hkv, D, seed):
    return (inputs.make_tensor(B, Sq, Hq, D, seed, inputs.Q), inputs.make_tensor(B, Sk, Hkv, D, seed, inputs.K),
            inputs.make_tensor(B, Sk, Hkv, D, seed, inputs.V))


def run_decode(q, k, v, causal, scale):
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device=q.device)
    need = binding.attn_decode_workspace_size(B, Sq, Sk, Hq, Hkv, D)
    assert need > 0
    ws = torch.full(((need + 3) // 4,), float("nan"), dtype=torch.float32, device=q.device)
    st = binding.attn_fwd_decode(q, k, v, o, lse, B, Sq, Sk, Hq, Hkv, D, int(causal), scale, ws, need, None)
    assert st == binding.ATTN_OK, binding.attn_status_string(st)
    torch.cuda.synchronize()
    return o, lse


# (B, Sq, Sk, Hq, Hkv, D, causal): single-token decode at LLaMA3-70B/8B head shapes, a few query rows, a chunk
# whose packed rows span several tiles, tails off the 64-key tiles, D = 64 / 256, non-causal
SHAPES = [
    (1, 1, 8192, 64, 8, 128, 1), (4, 1, 1000, 32, 8, 128, 1), (2, 3, 777, 32, 8, 64, 1), (1, 16, 4096, 64, 8, 256, 1),
    (3, 5, 300, 12, 3, 128, 0), (1, 1, 1, 8, 2, 128, 1), (2, 1, 64, 8, 8, 128, 1), (1, 100, 1000, 8, 2, 128, 1),
    (2, 7, 200, 16, 4, 128, 1), (1, 2, 65, 64, 8, 128, 1), (1, 33, 2048, 32, 8, 128, 1),
]


@pytest.mark.parametrize("B,Sq,Sk,Hq,Hkv,D,causal", SHAPES, ids=str)
def test_decode_shapes(B, Sq, Sk, Hq, Hkv, D, causal):
    tag = "decode B%d Sq%d Sk%d Hq%d Hkv%d D%d causal%d" % (B, Sq, Sk, Hq, Hkv, D, causal)
    U.say(tag)
    scale = 1.0 / math.sqrt(D)
    q, k, v = cpu_qkv(B, Sq, Sk, Hq, Hkv, D, seed=7000 + Sq + 3 * Sk + Hq + D)
    o, lse = run_decode(q.cuda(), k.cuda(), v.cuda(), bool(causal), scale)
    O, L = oracle_mod.attn_full(q.numpy(), k.numpy(), v.numpy(), bool(causal), scale)
    U.check(U.stats(o.cpu().numpy(), lse.cpu().numpy(), O, L), tag)


def test_decode_matches_regular_path():
    """Same inputs through attn_fwd_ex and attn_fwd_decode: equal within the attention tolerance."""
    B, Sq, Sk, Hq, Hkv, D = 8, 2, 3000, 64, 8, 128
    q, k, v = cpu_qkv(B, Sq, Sk, Hq, Hkv, D, seed=7101)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o1, l1 = run_decode(qd, kd, vd, True, inputs.SCALE_D128)
    o2, l2 = U.run(qd, kd, vd, True, inputs.SCALE_D128)
    e = (o1.float() - o2.float()).abs()
    assert float(e.max()) <= 4e-3 and float(e.mean()) <= 5e-4
    assert float((l1 - l2).abs().max()) <= 1e-3


def test_decode_convenience_and_negative_scale():
    B, Sq, Sk, Hq, Hkv, D = 2, 1, 500, 16, 4, 128
    q, k, v = cpu_qkv(B, Sq, Sk, Hq, Hkv, D, seed=7102)
    o, lse = binding.decode(q.cuda(), k.cuda(), v.cuda(), causal=True, scale=-0.05)
    torch.cuda.synchronize()
    O, L = oracle_mod.attn_full(q.numpy(), k.numpy(), v.numpy(), True, np.float32(-0.05).item())
    U.check(U.stats(o.cpu().numpy(), lse.cpu().numpy(), O, L), "decode convenience scale -0.05")


def test_decode_workspace_too_small_launches_nothing():
    B, Sq, Sk, Hq, Hkv, D = 1, 1, 256, 8, 2, 128
    q, k, v = cpu_qkv(B, Sq, Sk, Hq, Hkv, D, seed=7103)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o = torch.full_like(qd, float("nan"))
    need = binding.attn_decode_workspace_size(B, Sq, Sk, Hq, Hkv, D)
    ws = torch.empty(((need + 3) // 4,), dtype=torch.float32, device="cuda")
    st = binding.attn_fwd_decode(qd, kd, vd, o, None, B, Sq, Sk, Hq, Hkv, D, 1, 0.088, ws, need - 4, None)
    assert st == binding.ATTN_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool(torch.isnan(o).all().item())


def test_decode_on_a_non_default_stream_with_its_own_workspace():
    """binding.decode() allocating the workspace itself while launching on another stream (the workspace
    is then tied to that stream): the same bits as on the current stream."""
    B, Sq, Sk, Hq, Hkv, D = 2, 3, 2000, 32, 8, 128
    scale = 1.0 / math.sqrt(D)
    q, k, v = cpu_qkv(B, Sq, Sk, Hq, Hkv, D, seed=7101)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o1, l1 = binding.decode(qd, kd, vd, causal=True, scale=scale)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    o2, l2 = binding.decode(qd, kd, vd, causal=True, scale=scale, stream=s)
    s.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
