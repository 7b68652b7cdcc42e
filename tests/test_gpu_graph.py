"""HIP graph capture of libattn's entry points.

Each entry point is captured once into a torch CUDA graph (a HIP graph on ROCm) and replayed several times,
with eager work and device synchronisations between the replays.  Every replay must give the eager result
bit for bit, also after new data has been copied into the captured input buffers (the graph reads the
buffers live).  The library allocates nothing, issues no memset and makes no synchronising call on these
paths, so its kernel launches are all that a graph holds.
"""
import pytest
import torch

from dnn_compiler_pipelining_amd import binding, inputs
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module", autouse=True)
def gpu():
    U.require_gpu()


def qkv(B, Sq, Sk, Hq, Hkv, D, seed):
    return (inputs.make_tensor(B, Sq, Hq, D, seed, inputs.Q, "cuda"),
            inputs.make_tensor(B, Sk, Hkv, D, seed, inputs.K, "cuda"),
            inputs.make_tensor(B, Sk, Hkv, D, seed, inputs.V, "cuda"))


def capture(fn):
    """fn run once eagerly on a side stream, then captured into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def replay_and_check(g, outs, refs, busy, tag):
    """Replay g REPLAYS times; before each, the outputs are set to NaN (eagerly, outside the graph) and
    after each, unrelated eager work runs and the device synchronises; every replay must reproduce refs."""
    for r in range(REPLAYS):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        busy()
        torch.cuda.synchronize()
        for t, ref in zip(outs, refs):
            assert torch.equal(t, ref), "%s: replay %d differs from the eager result" % (tag, r)


def eager_noise():
    """Unrelated eager work between replays: an attention call on other data and a reduction."""
    q, k, v = qkv(1, 300, 300, 8, 2, 128, 77)
    U.run(q, k, v, True, inputs.SCALE_D128)
    torch.randn(1 << 20, device="cuda").sum().item()


@pytest.mark.parametrize("B,S,Hq,Hkv,causal,variant", [
    (2, 1000, 16, 2, 1, None),
    (1, 700, 8, 2, 0, None),
    (2, 333, 12, 3, 1, {"schedule": "serial4", "bn": 32}),
    (1, 650, 8, 2, 1, {"schedule": "overlap", "place": "front"}),
    (1, 257, 8, 1, 1, {"schedule": "pingpong"}),
    (2, 300, 8, 2, 1, {"schedule": "serial4_16"}),
], ids=str)
def test_forward_graph_replays(B, S, Hq, Hkv, causal, variant):
    tag = "forward B%d S%d Hq%d Hkv%d causal%d %s" % (B, S, Hq, Hkv, causal, variant)
    U.say("graph " + tag)
    sc = inputs.SCALE_D128
    q, k, v = qkv(B, S, S, Hq, Hkv, 128, 500 + S)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    o_ref, lse_ref = U.run(q, k, v, bool(causal), sc, variant)
    g = capture(lambda: binding.forward(q, k, v, causal=bool(causal), scale=sc, out=o, lse=lse, variant=variant))
    replay_and_check(g, (o, lse), (o_ref, lse_ref), eager_noise, tag)
    # new data in the captured buffers: the replay reads them live
    q2, k2, v2 = qkv(B, S, S, Hq, Hkv, 128, 600 + S)
    q.copy_(q2)
    k.copy_(k2)
    v.copy_(v2)
    o2_ref, lse2_ref = U.run(q2, k2, v2, bool(causal), sc, variant)
    assert not torch.equal(o2_ref, o_ref)
    replay_and_check(g, (o, lse), (o2_ref, lse2_ref), eager_noise, tag + " (new data)")


@pytest.mark.parametrize("B,Sq,Sk,Hq,Hkv,D", [(4, 1, 4096, 64, 8, 128), (2, 16, 3000, 32, 8, 64)], ids=str)
def test_decode_graph_replays(B, Sq, Sk, Hq, Hkv, D):
    """The split-KV path with a caller workspace and its no-allocation form on the library's own array,
    each captured: both launches of each (split kernel and combine kernel) replay to the eager bits."""
    tag = "decode B%d Sq%d Sk%d Hq%d Hkv%d D%d" % (B, Sq, Sk, Hq, Hkv, D)
    U.say("graph " + tag)
    sc = inputs.scale_for(D)
    q, k, v = qkv(B, Sq, Sk, Hq, Hkv, D, 700 + Sk)
    need = binding.attn_decode_workspace_size(B, Sq, Sk, Hq, Hkv, D)
    ws = torch.empty(((need + 3) // 4,), dtype=torch.float32, device="cuda")
    o_ref = torch.empty_like(q)
    lse_ref = torch.empty((B, Hq, Sq), dtype=torch.float32, device="cuda")
    st = binding.attn_fwd_decode(q, k, v, o_ref, lse_ref, B, Sq, Sk, Hq, Hkv, D, 1, sc, ws, need, None)
    assert st == binding.ATTN_OK, binding.attn_status_string(st)
    torch.cuda.synchronize()

    o = torch.empty_like(q)
    lse = torch.empty_like(lse_ref)

    def with_ws():
        s = torch.cuda.current_stream()
        assert binding.attn_fwd_decode(q, k, v, o, lse, B, Sq, Sk, Hq, Hkv, D, 1, sc, ws, need, s) == binding.ATTN_OK

    def static():
        s = torch.cuda.current_stream()
        assert binding.attn_fwd_decode_static(q, k, v, o, lse, B, Sq, Sk, Hq, Hkv, D, 1, sc, s) == binding.ATTN_OK

    for name, fn in (("caller workspace", with_ws), ("static workspace", static)):
        g = capture(fn)
        replay_and_check(g, (o, lse), (o_ref, lse_ref), eager_noise, "%s, %s" % (tag, name))
        del g


def test_gemm_graph_replays():
    M, N, K = 520, 392, 384
    U.say("graph gemm %dx%dx%d" % (M, N, K))
    for layout in (0, 1):
        a = inputs.make_matrix(M, K, 31, 0, device="cuda")
        b = inputs.make_matrix(K, N, 31, 1, device="cuda") if layout == 0 else \
            inputs.make_matrix(N, K, 31, 1, device="cuda")
        c_ref = torch.empty((M, N), dtype=torch.float16, device="cuda")
        assert binding.gemm_f16(a, b, c_ref, M, N, K, layout, None) == binding.ATTN_OK
        torch.cuda.synchronize()
        c = torch.empty_like(c_ref)
        g = capture(lambda: binding.gemm_f16(a, b, c, M, N, K, layout, torch.cuda.current_stream()))
        replay_and_check(g, (c,), (c_ref,), eager_noise, "gemm layout %d" % layout)
