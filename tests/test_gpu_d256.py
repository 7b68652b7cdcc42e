"""GPU parity of head dimension 256 (SERIAL4 schedule, one workgroup per CU) against the fp64 oracle, same bar as
tests/test_gpu_parity.py."""
import math

import numpy as np
import pytest
import torch

from dnn_compiler_pipelining_amd import binding, inputs
from oracle import oracle as oracle_mod
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

D = 256
SC = 1.0 / math.sqrt(D)


def cpu_qkv(B, Sq, Sk, Hq, Hkv, seed):
    return (inputs.make_tensor(B, Sq, Hq, D, seed, inputs.Q), inputs.make_tensor(B, Sk, Hkv, D, seed, inputs.K),
            inputs.make_tensor(B, Sk, Hkv, D, seed, inputs.V))


@pytest.fixture(scope="module", autouse=True)
def gpu():
    U.require_gpu()


# (B, Sq, Sk, Hq, Hkv, causal, scale)
SHAPES = [
    (1, 1, 1, 8, 2, 1, SC), (2, 63, 63, 8, 8, 1, SC), (1, 64, 64, 8, 1, 1, SC), (2, 65, 65, 8, 2, 0, SC),
    (1, 129, 129, 4, 4, 1, SC), (2, 200, 200, 16, 4, 1, SC), (1, 1000, 1000, 8, 2, 1, SC),
    (1, 1000, 1000, 8, 2, 0, SC), (1, 300, 300, 8, 2, 1, -SC), (3, 77, 77, 12, 3, 1, SC),
    (1, 100, 700, 8, 2, 1, SC), (2, 7, 300, 8, 2, 1, SC), (1, 333, 90, 8, 2, 0, SC), (1, 256, 256, 8, 2, 1, 0.0),
]


@pytest.mark.parametrize("B,Sq,Sk,Hq,Hkv,causal,scale", SHAPES, ids=lambda x: str(x))
def test_d256_shapes(B, Sq, Sk, Hq, Hkv, causal, scale):
    tag = "D256 B%d Sq%d Sk%d Hq%d Hkv%d causal%d scale%.4g" % (B, Sq, Sk, Hq, Hkv, causal, scale)
    U.say(tag)
    q, k, v = cpu_qkv(B, Sq, Sk, Hq, Hkv, seed=5000 + Sq + 5 * Sk + Hq)
    U.full_parity(q, k, v, bool(causal), scale, tag)


def test_d256_larger_sampled():
    """B=2, S=4096, 32 query heads on 8 KV heads, D=256: sampled rows of the first and last batch entries."""
    B, S, Hq, Hkv = 2, 4096, 32, 8
    U.say("D256 B%d S%d Hq%d Hkv%d sampled" % (B, S, Hq, Hkv))
    q, k, v = cpu_qkv(B, S, S, Hq, Hkv, seed=71)
    o, lse = U.run(q.cuda(), k.cuda(), v.cuda(), True, SC)
    U.whole_output_sane(o, lse)
    rng = np.random.default_rng(3)
    rows = U.sample_rows(S, rng, n_random=48)
    heads = list(range(0, Hq, 3)) + [Hq - 1]
    hs = np.repeat(np.array(heads, dtype=np.int32), len(rows))
    rs = np.tile(np.array(rows, dtype=np.int32), len(heads))
    for b in (0, B - 1):
        O, L = oracle_mod.attn_rows(q[b].numpy(), k[b].numpy(), v[b].numpy(), hs, rs, True, SC)
        rows_t = torch.as_tensor(rs, dtype=torch.long, device=o.device)
        heads_t = torch.as_tensor(hs, dtype=torch.long, device=o.device)
        st = U.stats(o[b][rows_t, heads_t].cpu().numpy(), lse[b][heads_t, rows_t].cpu().numpy(), O, L)
        U.check(st, "D256 B%d S%d batch %d" % (B, S, b))


def test_d256_variants_bitwise_identical():
    """Ring depth and workgroup order give the same bits at D=256 (serial4, its only schedule); the other
    schedules are refused with ATTN_ERR_UNSUPPORTED and launch nothing."""
    q, k, v = cpu_qkv(1, 700, 700, 8, 2, seed=72)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o1, l1 = U.run(qd, kd, vd, True, SC)
    for sched in ("serial4",):
        for ring in (2, 4):
            for xcd, lpt in ((0, 0), (1, 1)):
                var = {"schedule": sched, "ring": ring, "xcd": xcd, "lpt": lpt}
                o2, l2 = U.run(qd, kd, vd, True, SC, var)
                assert torch.equal(o1, o2) and torch.equal(l1, l2), var
    for sched in sorted(set(binding.SCHEDULES) - set(("serial4",))):
        o = torch.full_like(qd, float("nan"))
        st = binding.attn_fwd_variant(qd, kd, vd, o, None, 1, 700, 700, 8, 2, 256, 1, SC, binding.SCHEDULES[sched],
                                      -1, -1, -1, -1, -1, -1, None)
        assert st == binding.ATTN_ERR_UNSUPPORTED, sched
        torch.cuda.synchronize()
        assert bool(torch.isnan(o).all().item()), sched
