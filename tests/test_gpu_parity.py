"""GPU parity: libattn (through the C ABI) against the fp64 oracle on identical seeded inputs.

Bar: max |O_gpu - O_ref| <= 4e-3, mean <= 5e-4 over the compared O elements, max |LSE error| <= 1e-3,
no NaN/Inf.  Small shapes are compared element by element over the whole output; the full-size
workloads in the launch configuration the benchmark times are compared on sampled rows (all heads,
first/last batch entries, tile edges, random rows) that the oracle computes one by one.
"""
import numpy as np
import pytest
import torch

from dnn_compiler_pipelining_amd import binding, inputs
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

D = 128
SC = inputs.SCALE_D128


def cpu_qkv(B, S, Hq, Hkv, seed):
    return (inputs.make_tensor(B, S, Hq, D, seed, inputs.Q), inputs.make_tensor(B, S, Hkv, D, seed, inputs.K),
            inputs.make_tensor(B, S, Hkv, D, seed, inputs.V))


@pytest.fixture(scope="module", autouse=True)
def gpu():
    U.require_gpu()


# (B, S, Hq, Hkv, causal, scale): S spans 1, tile edges (64, 128) and ragged tails; g = 1, 2, 3, 4, 8.
EDGE = [
    (1, 1, 8, 2, 1, SC), (1, 1, 8, 2, 0, SC), (2, 2, 8, 2, 1, SC), (1, 63, 8, 8, 1, SC), (1, 64, 8, 1, 1, SC),
    (2, 65, 8, 2, 0, SC), (1, 127, 6, 2, 1, SC), (1, 128, 4, 4, 0, SC), (1, 129, 8, 1, 1, SC),
    (2, 200, 16, 4, 1, SC), (1, 257, 2, 1, 1, SC), (1, 384, 32, 8, 1, SC), (1, 1000, 8, 2, 1, SC),
    (1, 1000, 8, 2, 0, SC), (1, 300, 8, 2, 1, -SC), (1, 300, 8, 2, 1, 0.0), (1, 300, 8, 2, 0, 0.25),
    (3, 77, 12, 3, 1, SC),
    # scale 1 and 0.7: scores of standard deviation 11 and 8, sharply peaked rows whose running max rises
    # often, so the sum-checked rescale takes its rare path many times per row
    (1, 2048, 8, 2, 1, 1.0), (1, 1500, 16, 2, 0, 0.7),
]


@pytest.mark.parametrize("B,S,Hq,Hkv,causal,scale", EDGE, ids=lambda x: str(x))
def test_edge_shapes(B, S, Hq, Hkv, causal, scale):
    tag = "B%d S%d Hq%d Hkv%d causal%d scale%.4g" % (B, S, Hq, Hkv, causal, scale)
    U.say("edge " + tag)
    q, k, v = cpu_qkv(B, S, Hq, Hkv, seed=1000 + S + 7 * Hq + Hkv)
    U.full_parity(q, k, v, bool(causal), scale, tag)


def test_workload_small_full():
    """The 8B-shaped B=1 S=512 workload, whole output against the oracle; and the errors are at the level
    of the kernel's own arithmetic (tests/test_tolerance_model.py: round-to-nearest P and O give
    max |dLSE| about 1.5e-4 on such inputs, truncation over 3e-4), not merely inside the bar."""
    w = inputs.WORKLOADS[0]
    U.say("workload " + w.name)
    q, k, v = inputs.make_inputs(w, "cpu")
    st = U.full_parity(q, k, v, w.causal, w.scale, w.name)
    assert st["max_lse"] <= 3e-4 and st["max_o"] <= 2e-3, st


@pytest.mark.parametrize("idx", [1, 2], ids=lambda i: inputs.WORKLOADS[i].name)
def test_workload_full_output(idx):
    """The B = 1, S = 8192 workloads (LLaMA3-8B and -70B heads): every output row of every head against
    the oracle."""
    w = inputs.WORKLOADS[idx]
    U.say("workload %s (full size, whole output)" % w.name)
    q, k, v = inputs.make_inputs(w, "cpu")
    U.full_parity(q, k, v, w.causal, w.scale, w.name + " whole output")


@pytest.mark.parametrize("idx", [3, 4], ids=lambda i: inputs.WORKLOADS[i].name)
def test_workload_full_size_sampled(idx):
    """The B = 64 workloads at full size: sampled rows of every third head of three batch entries, and
    three whole (batch, head) slices (every query row of that head)."""
    w = inputs.WORKLOADS[idx]
    U.say("workload %s (full size, sampled rows and whole slices)" % w.name)
    q, k, v = inputs.make_inputs(w, "cuda")
    o, lse = U.run(q, k, v, w.causal, w.scale)
    U.whole_output_sane(o, lse)
    batches = sorted({0, w.B // 2, w.B - 1})
    heads = list(range(0, w.Hq, 3)) + [w.Hq - 1]
    U.sampled_parity(w, q, k, v, o, lse, batches, heads=heads, n_random=64, tag=w.name)
    for b, h in ((0, 0), (w.B // 2, w.Hq // 2 + 1), (w.B - 1, w.Hq - 1)):
        U.slice_parity(w, q, k, v, o, lse, b, h, tag="%s slice b%d h%d" % (w.name, b, h))
    del q, k, v, o, lse
    torch.cuda.empty_cache()


@pytest.mark.parametrize("half", [0, 1])
def test_b64_s2048_whole_output(half):
    """llama3-8b_b64_s2048 at full size, in the launch the bench times: every one of its 537M outputs (all
    64 batch entries, every row, head and d) against the oracle, half of the batch entries per case."""
    w = inputs.WORKLOADS[3]
    U.say("workload %s (full size, whole output of batch entries %d..%d)" % (w.name, half * 32, half * 32 + 31))
    q, k, v = inputs.make_inputs(w, "cuda")
    o, lse = U.run(q, k, v, w.causal, w.scale)
    batches = list(range(half * w.B // 2, (half + 1) * w.B // 2))
    st = U.batch_entries_parity(w, q, k, v, o, lse, batches, tag="%s batch entries %d..%d" %
                                (w.name, batches[0], batches[-1]))
    assert st["n"] == w.B // 2 * w.S * w.Hq * w.D
    del q, k, v, o, lse
    torch.cuda.empty_cache()


@pytest.mark.parametrize("b", [0, 21, 42, 63])
def test_b64_s8192_whole_batch_entry(b):
    """llama3-70b_b64_s8192 at full size, in the launch the bench times: every output of one batch entry
    (67M outputs) against the oracle; the four cases take the first, the last and two between."""
    w = inputs.WORKLOADS[4]
    U.say("workload %s (full size, whole batch entry %d)" % (w.name, b))
    q, k, v = inputs.make_inputs(w, "cuda")
    o, lse = U.run(q, k, v, w.causal, w.scale)
    U.batch_entries_parity(w, q, k, v, o, lse, [b], tag="%s batch entry %d" % (w.name, b))
    del q, k, v, o, lse
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", [w.name for w in inputs.VARIANT_SHAPES])
def test_variant_shapes_full_size_sampled(name):
    """The attention variant shapes the bench times (non-causal, sequence lengths off the tiles, chunked
    prefill, D = 64 and 256), at full size in the tuned launch: every output finite and |O| within
    max |V|, and sampled rows of every fifth head of the first and last batch entries against the
    oracle."""
    w = inputs.VARIANT_BY_NAME[name]
    U.say("variant shape %s (full size, sampled rows)" % w.name)
    q, k, v = inputs.make_variant_inputs(w, "cuda")
    o = torch.full_like(q, float("nan"))
    lse = torch.full((w.B, w.Hq, w.Sq), float("nan"), dtype=torch.float32, device=q.device)
    binding.forward(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse)
    torch.cuda.synchronize()
    U.whole_output_sane(o, lse)
    heads = list(range(0, w.Hq, 5)) + [w.Hq - 1]
    U.sampled_parity_shape(w, q, k, v, o, lse, [0, w.B - 1], heads, tag=w.name)
    del q, k, v, o, lse
    torch.cuda.empty_cache()


def test_noncausal_full_length_sampled():
    """Non-causal attention at the bench workload's head shape and sequence length (B = 2): every row sees
    all 128 key tiles, the path the causal workloads take only for their last rows.  Sampled rows of every
    fourth head of both batch entries, and one whole (batch, head) slice."""
    w = inputs.Workload("noncausal_b2_s8192", 2, 8192, 64, 8, 128, False, 31)
    U.say("non-causal B2 S8192 Hq64 Hkv8 (sampled rows and one slice)")
    q, k, v = inputs.make_inputs(w, "cuda")
    o, lse = U.run(q, k, v, w.causal, w.scale)
    U.whole_output_sane(o, lse)
    U.sampled_parity(w, q, k, v, o, lse, [0, 1], heads=list(range(0, w.Hq, 4)) + [w.Hq - 1], n_random=32,
                     tag=w.name)
    U.slice_parity(w, q, k, v, o, lse, 1, 37, tag="%s slice b1 h37" % w.name)
    del q, k, v, o, lse
    torch.cuda.empty_cache()


def test_first_causal_row_is_v0_bitwise():
    q, k, v = cpu_qkv(2, 333, 16, 4, seed=77)
    o, _ = U.run(q.cuda(), k.cuda(), v.cuda(), True, SC)
    g = 4
    want = v[:, 0].repeat_interleave(g, dim=1)  # [B, Hq, D]
    assert torch.equal(o[:, 0].cpu(), want)


def test_zero_q_gives_prefix_means():
    B, S, Hq, Hkv = 1, 300, 8, 2
    _, k, v = cpu_qkv(B, S, Hq, Hkv, seed=78)
    q = torch.zeros(B, S, Hq, D, dtype=torch.float16)
    o, lse = U.run(q.cuda(), k.cuda(), v.cuda(), True, SC)
    vd = v.double()
    pref = vd.cumsum(dim=1) / torch.arange(1, S + 1, dtype=torch.float64).view(1, S, 1, 1)
    want = pref.repeat_interleave(Hq // Hkv, dim=2)
    err = (o.cpu().double() - want).abs() - 2.0 ** -10 * want.abs()
    assert err.max().item() <= 1e-6
    want_lse = torch.log(torch.arange(1, S + 1, dtype=torch.float64)).view(1, 1, S).expand(B, Hq, S)
    assert (lse.cpu().double() - want_lse).abs().max().item() <= 1e-5


def test_constant_v_rows():
    B, S, Hq, Hkv = 2, 260, 8, 2
    q, k, _ = cpu_qkv(B, S, Hq, Hkv, seed=79)
    u = torch.randn(B, 1, Hkv, D, generator=torch.Generator().manual_seed(5)).to(torch.float16)
    v = u.expand(B, S, Hkv, D).contiguous()
    for causal in (True, False):
        o, _ = U.run(q.cuda(), k.cuda(), v.cuda(), causal, SC)
        want = u.double().repeat_interleave(Hq // Hkv, dim=2).expand(B, S, Hq, D)
        err = (o.cpu().double() - want).abs() / want.abs().clamp_min(1e-3)
        assert err.max().item() <= 2.0 ** -9


def test_gqa_head_map():
    """KV head c holds the constant c+1: query head h must return floor(h / g) + 1."""
    for Hq, Hkv in ((32, 8), (64, 8), (12, 3), (8, 8)):
        B, S = 1, 200
        q, k, _ = cpu_qkv(B, S, Hq, Hkv, seed=80 + Hq)
        v = torch.empty(B, S, Hkv, D, dtype=torch.float16)
        for c in range(Hkv):
            v[:, :, c] = c + 1
        o, _ = U.run(q.cuda(), k.cuda(), v.cuda(), True, SC)
        g = Hq // Hkv
        want = (torch.arange(Hq) // g + 1).double().view(1, 1, Hq, 1)
        err = (o.cpu().double() - want).abs() / want
        assert err.max().item() <= 2.0 ** -9, (Hq, Hkv)


def test_deterministic_and_lse_optional():
    w = inputs.WORKLOADS[0]
    q, k, v = inputs.make_inputs(w, "cuda")
    o1, l1 = U.run(q, k, v, True, w.scale)
    o2, l2 = U.run(q, k, v, True, w.scale)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o3 = torch.full_like(q, float("nan"))
    binding.forward(q, k, v, causal=True, scale=w.scale, out=o3, want_lse=False)
    torch.cuda.synchronize()
    assert torch.equal(o1, o3)


def test_non_default_stream():
    w = inputs.WORKLOADS[0]
    q, k, v = inputs.make_inputs(w, "cuda")
    o1, l1 = U.run(q, k, v, True, w.scale)
    s = torch.cuda.Stream()
    o2 = torch.full_like(q, float("nan"))
    l2 = torch.full_like(l1, float("nan"))
    torch.cuda.synchronize()
    st = binding.attn_fwd_stream(q, k, v, o2, l2, w.B, w.S, w.Hq, w.Hkv, w.D, 1, w.scale, s)
    assert st == binding.ATTN_OK
    s.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_raw_c_entry_point_null_stream():
    """attn_fwd (null stream) with raw device addresses."""
    q, k, v = cpu_qkv(1, 130, 8, 2, seed=81)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((1, 8, 130), float("nan"), device="cuda")
    torch.cuda.synchronize()
    st = binding.attn_fwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(),
                          1, 130, 8, 2, 128, 1, SC)
    assert st == binding.ATTN_OK
    torch.cuda.synchronize()
    from oracle import oracle as oracle_mod
    O, L = oracle_mod.attn_full(q.numpy(), k.numpy(), v.numpy(), True, SC)
    U.check(U.stats(o.cpu().numpy(), lse.cpu().numpy(), O, L), "raw attn_fwd")


def test_gpu_validation_errors_launch_nothing():
    q, k, v = cpu_qkv(1, 64, 8, 2, seed=82)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o = torch.full_like(qd, float("nan"))
    st = binding.attn_fwd(qd, kd, vd, o, None, 1, 64, 8, 2, 96, 1, SC)
    assert st == binding.ATTN_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool(torch.isnan(o).all().item())


# S = 1, 33 and 64 give a single key tile: the overlap and ping-pong schedules take their n_tiles == 1
# paths there; 8192 is the bench workload's sequence length
@pytest.mark.parametrize("B,S,Hq,Hkv,causal", [(1, 1000, 8, 2, 1), (2, 333, 16, 4, 0), (1, 257, 6, 2, 1),
                                               (1, 1, 8, 2, 1), (2, 33, 8, 2, 1), (1, 64, 16, 4, 0),
                                               (1, 64, 8, 1, 1), (1, 130, 12, 3, 1), (1, 8192, 64, 8, 1)], ids=str)
def test_schedules_bitwise_identical(B, S, Hq, Hkv, causal):
    """The tile schedules against each other: each accumulator sees the same arithmetic in the same order,
    so any LDS race (a slot rewritten while another wave still reads it) would show up as a difference."""
    q, k, v = cpu_qkv(B, S, Hq, Hkv, seed=90 + S)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    U.say("schedules B%d S%d Hq%d Hkv%d causal%d" % (B, S, Hq, Hkv, causal))
    o1, l1 = U.run(qd, kd, vd, bool(causal), SC, {"bn": 64})
    for sched in U.SCHEDULES_D128:
        o2, l2 = U.run(qd, kd, vd, bool(causal), SC, {"schedule": sched, "bn": 64})
        assert torch.equal(o1, o2) and torch.equal(l1, l2), sched


@pytest.mark.parametrize("B,S,Hq,Hkv,causal", [(1, 700, 8, 2, 1), (2, 257, 12, 3, 0)], ids=str)
def test_all_variants_bitwise_identical(B, S, Hq, Hkv, causal):
    """Every point of the searched variant space of one tile size (schedule x prefetch depth x workgroup
    order x placement x heads per workgroup) gives the same bits: 64-key tiles over every 32 x 32 x 16
    schedule, 32- and 128-key tiles over the serial schedules, and the 16 x 16 x 32 schedule's variants,
    each group against its own first point."""
    q, k, v = cpu_qkv(B, S, Hq, Hkv, seed=95 + S)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    for bn, scheds in ((64, U.SCHEDULES_D128), (32, ("serial", "serial4")), (128, ("serial", "serial4")),
                       (64, ("serial4_16",))):
        # the 16 x 16 x 32 schedule rounds differently: its variants are compared among themselves
        first = "serial4_16" if scheds == ("serial4_16",) else "serial"
        o1, l1 = U.run(qd, kd, vd, bool(causal), SC, {"schedule": first, "bn": bn})
        for sched in scheds:
            for ring in (2, 4):
                for xcd in (0, 1):
                    for lpt in (0, 1):
                        for place in (binding.PLACES if sched in ("wide", "overlap") else ("even",)):
                            for hpw in ((4, 2, 1) if sched == "wide" else (0,)):
                                var = {"schedule": sched, "ring": ring, "xcd": xcd, "lpt": lpt, "place": place,
                                       "bn": bn, "hpw": hpw}
                                o2, l2 = U.run(qd, kd, vd, bool(causal), SC, var)
                                assert torch.equal(o1, o2) and torch.equal(l1, l2), var


# Every compiled D = 128 kernel instance (schedule x ring depth x softmax placement x keys per tile) on its
# own against the oracle, causal with ragged tails and non-causal, so a fault confined to one instance is
# named.
INSTANCES = ([(sched, ring, place, 64) for sched in U.SCHEDULES_D128 for ring in (2, 4)
              for place in (binding.PLACES if sched in ("wide", "overlap") else ("even",))] +
             [(sched, ring, "even", bn) for sched in ("serial", "serial4") for ring in (2, 4) for bn in (32, 128)] +
             [("serial4_16", ring, "even", 64) for ring in (2, 4)])


@pytest.mark.parametrize("sched,ring,place,bn", INSTANCES, ids=lambda x: str(x))
# GQA ratios 4, 3, 2 and 8: the 64-row kernel's workgroups then take 4 heads, 1 head x 256 rows, 2 heads x 128
# rows, and 4 of 8 heads (two workgroups per KV head)
@pytest.mark.parametrize("B,S,Hq,Hkv,causal", [(1, 650, 8, 2, 1), (2, 201, 12, 4, 0), (1, 300, 4, 2, 1),
                                               (1, 333, 16, 2, 1)], ids=str)
def test_every_instance_against_oracle(B, S, Hq, Hkv, causal, sched, ring, place, bn):
    tag = "instance %s ring%d %s bn%d B%d S%d Hq%d Hkv%d causal%d" % (sched, ring, place, bn, B, S, Hq, Hkv,
                                                                      causal)
    U.say(tag)
    q, k, v = cpu_qkv(B, S, Hq, Hkv, seed=300 + S + Hq)
    U.full_parity(q, k, v, bool(causal), SC, tag,
                  {"schedule": sched, "ring": ring, "xcd": 1, "lpt": 1, "place": place, "bn": bn})


@pytest.mark.parametrize("hpw", [4, 2, 1])
@pytest.mark.parametrize("B,S,Hq,Hkv,causal", [(1, 650, 8, 2, 1), (2, 201, 12, 4, 0), (1, 333, 16, 2, 1),
                                               (1, 300, 6, 2, 1)], ids=str)
def test_wide_heads_per_workgroup_against_oracle(B, S, Hq, Hkv, causal, hpw):
    """The 64-row kernel with 4, 2 or 1 query heads per workgroup (64, 128 or 256 query rows of each),
    GQA ratios 4, 3 and 8 (with 3 and hpw 2 or 4, a workgroup's last waves fall past the group's heads)."""
    tag = "wide hpw%d B%d S%d Hq%d Hkv%d causal%d" % (hpw, B, S, Hq, Hkv, causal)
    U.say(tag)
    q, k, v = cpu_qkv(B, S, Hq, Hkv, seed=320 + S + Hq)
    U.full_parity(q, k, v, bool(causal), SC, tag, {"schedule": "wide", "hpw": hpw})


@pytest.mark.parametrize("sched,bn", [("serial4_16", 64), ("serial4", 32), ("serial", 32), ("serial4", 128)],
                         ids=str)
@pytest.mark.parametrize("scale", [-SC, 0.0, 1.0], ids=["neg", "zero", "one"])
def test_other_instances_at_edge_scales(sched, bn, scale):
    """The instances whose rounding differs from the 64-key 32 x 32 x 16 schedules, at a negative scale
    (Q negated in the kernel), zero (uniform weights) and 1 (sharply peaked rows: the rescale path runs
    many times per row), against the oracle."""
    tag = "%s bn%d scale %.4g" % (sched, bn, scale)
    U.say("edge scale " + tag)
    q, k, v = cpu_qkv(1, 700, 8, 2, seed=330)
    U.full_parity(q, k, v, True, scale, tag, {"schedule": sched, "bn": bn})


def tuned_entries():
    """(B, Sq, Sk, Hq, Hkv, variant) rows of the compiled-in tuned table."""
    import os
    import re

    from dnn_compiler_pipelining_amd import build
    text = open(os.path.join(build.CSRC, "tuned_table.h")).read()
    rows = re.findall(r"\{(\d+), (\d+), (\d+), (\d+), (\d+), \{SCHEDULE_(\w+), (\d), (\d), (\d), PLACE_(\w+), "
                      r"(\d+), (\d)\}", text)
    assert rows
    return [tuple(int(x) for x in r[:5]) + ({"schedule": r[5].lower(), "ring": int(r[6]), "xcd": int(r[7]),
                                             "lpt": int(r[8]), "place": r[9].lower(), "bn": int(r[10]),
                                             "hpw": int(r[11])},)
            for r in rows]


@pytest.mark.parametrize("entry", tuned_entries(), ids=lambda e: "B%d_S%d_Hq%d" % (e[0], e[1], e[3]))
def test_tuned_entries(entry):
    """Each tuned-table entry: the library reports that variant for the entry's own shape, and the variant
    matches the oracle on a shortened problem with the entry's heads (B = 1, a ragged S)."""
    B, Sq, Sk, Hq, Hkv, var = entry
    assert binding.attn_tuned_variant(B, Sq, Sk, Hq, Hkv, D) == var
    S = min(Sq, 777)
    U.say("tuned entry %s at S%d" % (var, S))
    q, k, v = cpu_qkv(1, S, Hq, Hkv, seed=400 + Hq)
    U.full_parity(q, k, v, True, SC, "tuned %s" % var, var)


def spiked_qkv(S, Hq, Hkv, hd, seed, spikes):
    """Q shifted by +1 per element, and at each (position j, c) every K head's row j set to the constant
    c * 128 / hd: key j then scores about 16 c log2 units above the N(0,1) keys for every query, so the
    tile sum check fires part-way through each row that sees it (the running max is raised after the
    first tile, the rare path of the online softmax), and before the redo the largest P overflow fp16."""
    q = inputs.make_tensor(1, S, Hq, hd, seed, inputs.Q)
    k = inputs.make_tensor(1, S, Hkv, hd, seed, inputs.K)
    v = inputs.make_tensor(1, S, Hkv, hd, seed, inputs.V)
    q = (q.float() + 1.0).half()
    for j, c in spikes:
        k[:, j] = c * 128.0 / hd
    return q, k, v


@pytest.mark.parametrize("hd", [128, 64, 256], ids=lambda x: "D%d" % x)
@pytest.mark.parametrize("causal", [1, 0], ids=lambda x: "causal%d" % x)
def test_running_max_raised_mid_row(hd, causal):
    """Keys 400 and 800 (tiles 6 and 12) score far above everything before them: parity with the oracle,
    the same bits from every schedule the head dimension runs, and the split-KV path on the last rows."""
    q, k, v = spiked_qkv(1000, 8, 2, hd, seed=77, spikes=[(400, 1.0), (800, 2.0)])
    tag = "spiked D%d causal%d" % (hd, causal)
    U.say(tag)
    U.full_parity(q, k, v, bool(causal), SC, tag)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o1, l1 = U.run(qd, kd, vd, bool(causal), SC)
    scheds = U.SCHEDULES_D128 if hd == 128 else ("serial", "serial4") if hd == 64 else ("serial4",)
    for sched in scheds:
        o2, l2 = U.run(qd, kd, vd, bool(causal), SC, sched)
        assert torch.equal(o1, o2) and torch.equal(l1, l2), sched
    # the last 4 query rows through the split-KV path against the same rows of the regular path, with
    # the planned splits and with splits of 8 tiles (512 keys), which put both spikes inside a split
    qt = qd[:, -4:].contiguous()
    ot, lt = torch.empty_like(qt), torch.empty((1, 8, 4), dtype=torch.float32, device=qt.device)
    binding.forward(qt, kd, vd, causal=bool(causal), scale=SC, out=ot, lse=lt)
    for split_tiles in (0, 8):
        od, ld = binding.decode(qt, kd, vd, causal=bool(causal), scale=SC, split_tiles=split_tiles)
        torch.cuda.synchronize()
        assert float((od.float() - ot.float()).abs().max()) <= U.MAX_ABS_O, split_tiles
        assert float((ld - lt).abs().max()) <= U.MAX_ABS_LSE, split_tiles
