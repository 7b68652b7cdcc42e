"""GPU parity of attn_fwd_ex: Sq query rows against Sk keys (chunked prefill), against the fp64 oracle.

With causal = 1 the mask is aligned at the bottom right (query row i attends keys 0..i + Sk - Sq).
Same bar as tests/test_gpu_parity.py.
"""
import numpy as np
import pytest
import torch

from dnn_compiler_pipelining_amd import binding, inputs
from oracle import oracle as oracle_mod
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

D = 128
SC = inputs.SCALE_D128


def cpu_qkv(B, Sq, Sk, Hq, Hkv, seed):
    return (inputs.make_tensor(B, Sq, Hq, D, seed, inputs.Q), inputs.make_tensor(B, Sk, Hkv, D, seed, inputs.K),
            inputs.make_tensor(B, Sk, Hkv, D, seed, inputs.V))


@pytest.fixture(scope="module", autouse=True)
def gpu():
    U.require_gpu()


# (B, Sq, Sk, Hq, Hkv, causal, scale): one query row, tails off the 64/128 tiles, offsets that are and are
# not multiples of the tile sizes, GQA ratios 1..8, non-causal with Sq > Sk.
RECT = [
    (1, 1, 64, 8, 2, 1, SC), (1, 1, 1000, 8, 2, 1, SC), (2, 7, 200, 8, 2, 1, SC), (1, 100, 300, 8, 8, 1, SC),
    (1, 128, 512, 16, 4, 1, SC), (1, 200, 1000, 8, 2, 1, SC), (2, 65, 129, 4, 1, 1, SC), (3, 129, 257, 12, 3, 1, SC),
    (1, 300, 301, 8, 2, 1, SC), (1, 50, 700, 8, 2, 0, SC), (1, 500, 37, 8, 2, 0, SC), (1, 256, 640, 8, 1, 1, -SC),
    (1, 64, 192, 8, 2, 1, 0.0),
]


@pytest.mark.parametrize("B,Sq,Sk,Hq,Hkv,causal,scale", RECT, ids=lambda x: str(x))
def test_rect_shapes(B, Sq, Sk, Hq, Hkv, causal, scale):
    tag = "B%d Sq%d Sk%d Hq%d Hkv%d causal%d scale%.4g" % (B, Sq, Sk, Hq, Hkv, causal, scale)
    U.say("rect " + tag)
    q, k, v = cpu_qkv(B, Sq, Sk, Hq, Hkv, seed=2000 + Sq + 3 * Sk + Hq)
    U.full_parity(q, k, v, bool(causal), scale, tag)


def test_chunked_prefill_llama3_70b_sampled():
    """A 2048-row chunk against an 8192-key cache at LLaMA3-70B head shapes, sampled rows, all heads."""
    B, Sq, Sk, Hq, Hkv = 1, 2048, 8192, 64, 8
    U.say("chunked prefill B%d Sq%d Sk%d Hq%d Hkv%d" % (B, Sq, Sk, Hq, Hkv))
    q, k, v = cpu_qkv(B, Sq, Sk, Hq, Hkv, seed=31)
    o, lse = U.run(q.cuda(), k.cuda(), v.cuda(), True, SC)
    U.whole_output_sane(o, lse)
    rng = np.random.default_rng(7)
    rows = U.sample_rows(Sq, rng, n_random=48)
    heads = list(range(0, Hq, 5)) + [Hq - 1]
    hs = np.repeat(np.array(heads, dtype=np.int32), len(rows))
    rs = np.tile(np.array(rows, dtype=np.int32), len(heads))
    O, L = oracle_mod.attn_rows(q[0].numpy(), k[0].numpy(), v[0].numpy(), hs, rs, True, SC)
    rows_t = torch.as_tensor(rs, dtype=torch.long, device=o.device)
    heads_t = torch.as_tensor(hs, dtype=torch.long, device=o.device)
    st = U.stats(o[0][rows_t, heads_t].cpu().numpy(), lse[0][heads_t, rows_t].cpu().numpy(), O, L)
    U.check(st, "chunked prefill 70B Sq2048 Sk8192")


@pytest.mark.parametrize("Sq,Sk", [(128, 512), (256, 1000), (384, 8192)], ids=str)
def test_chunk_equals_suffix_of_square_bitwise(Sq, Sk):
    """When Sk - Sq is a multiple of the 128-row query tile, the chunk's query tiles line up with the last
    tiles of the square Sk x Sk problem, so the kernel must produce the same bits for those rows."""
    if (Sk - Sq) % 128 != 0:
        Sk = Sq + 128 * ((Sk - Sq) // 128)
    B, Hq, Hkv = 1, 16, 2
    q, k, v = cpu_qkv(B, Sq, Sk, Hq, Hkv, seed=41 + Sq)
    pad = inputs.make_tensor(B, Sk - Sq, Hq, D, 43, inputs.Q)
    qfull = torch.cat([pad, q], dim=1).contiguous()
    o1, l1 = U.run(q.cuda(), k.cuda(), v.cuda(), True, SC, {"bn": 64})
    o2, l2 = U.run(qfull.cuda(), k.cuda(), v.cuda(), True, SC, {"bn": 64})
    assert torch.equal(o1, o2[:, Sk - Sq:]) and torch.equal(l1, l2[:, :, Sk - Sq:])


# (B, Sq, Sk, Hq, Hkv, causal): bottom-right offsets that are and are not multiples of the tiles, and
# Sk <= 64 (a single key tile) where the overlap and ping-pong schedules take their n_tiles == 1 paths
RECT = [(1, 333, 1100, 16, 4, 1), (1, 333, 1100, 16, 4, 0), (2, 1, 64, 8, 2, 1), (1, 17, 40, 8, 8, 1),
        (1, 64, 64, 4, 1, 0), (1, 100, 63, 8, 2, 0), (1, 129, 700, 12, 3, 1)]


@pytest.mark.parametrize("B,Sq,Sk,Hq,Hkv,causal", RECT, ids=str)
def test_rect_schedules_bitwise_identical(B, Sq, Sk, Hq, Hkv, causal):
    q, k, v = cpu_qkv(B, Sq, Sk, Hq, Hkv, seed=51 + Sq + Sk)
    tag = "rect B%d Sq%d Sk%d Hq%d Hkv%d causal%d" % (B, Sq, Sk, Hq, Hkv, causal)
    U.say(tag)
    st = U.full_parity(q, k, v, bool(causal), SC, tag)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o1, l1 = U.run(qd, kd, vd, bool(causal), SC, {"bn": 64})
    for sched in U.SCHEDULES_D128:
        o2, l2 = U.run(qd, kd, vd, bool(causal), SC, {"schedule": sched, "bn": 64})
        assert torch.equal(o1, o2) and torch.equal(l1, l2), sched
    assert st["finite"]


@pytest.mark.parametrize("sched,bn", [(s, bn) for s in ("serial", "serial4") for bn in (32, 128)] +
                         [("serial4_16", 64)], ids=str)
@pytest.mark.parametrize("B,Sq,Sk,Hq,Hkv,causal", RECT, ids=str)
def test_rect_tile_sizes_against_oracle(B, Sq, Sk, Hq, Hkv, causal, sched, bn):
    """32- and 128-key tiles of the serial schedules on the rectangular shapes: offsets that are not
    multiples of the tile, a single partial tile (Sk 40, 63), and Sk 64 (two 32-key tiles, or half of one
    128-key tile)."""
    q, k, v = cpu_qkv(B, Sq, Sk, Hq, Hkv, seed=61 + Sq + Sk)
    tag = "rect %s bn%d B%d Sq%d Sk%d Hq%d Hkv%d causal%d" % (sched, bn, B, Sq, Sk, Hq, Hkv, causal)
    U.say(tag)
    U.full_parity(q, k, v, bool(causal), SC, tag, {"schedule": sched, "bn": bn})


def test_ex_validation_launches_nothing():
    q, k, v = cpu_qkv(1, 65, 64, 8, 2, seed=52)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o = torch.full_like(qd, float("nan"))
    st = binding.attn_fwd_ex(qd, kd, vd, o, None, 1, 65, 64, 8, 2, 128, 1, SC, None)
    assert st == binding.ATTN_ERR_SHAPE
    torch.cuda.synchronize()
    assert bool(torch.isnan(o).all().item())
