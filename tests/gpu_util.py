"""Helpers shared by the GPU parity tests: run libattn, compare with the fp64 oracle."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

from dnn_compiler_pipelining_amd import binding, inputs
from oracle import oracle as oracle_mod

# Every tile schedule at head dimension 128 (binding.SCHEDULES); all give bitwise identical results.
SCHEDULES_D128 = ("serial", "overlap", "pingpong", "serial4", "wide")

# Parity bar for fp16 outputs against the fp64 oracle.
MAX_ABS_O = 4e-3
MEAN_ABS_O = 5e-4
MAX_ABS_LSE = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU test run without a visible GPU")
    binding.load()  # raises if libattn.so is missing: no fallback


def run(q, k, v, causal, scale, variant=None):
    """q/k/v on the GPU.  Outputs are pre-filled with NaN so unwritten elements fail.  `variant` names a
    kernel variant (binding.variant_fields); None runs the tuned one."""
    o = torch.full_like(q, float("nan"))
    B, S, Hq, _ = q.shape
    lse = torch.full((B, Hq, S), float("nan"), dtype=torch.float32, device=q.device)
    binding.forward(q, k, v, causal=causal, scale=scale, out=o, lse=lse, variant=variant)
    torch.cuda.synchronize()
    return o, lse


def stats(o_gpu: np.ndarray, lse_gpu: np.ndarray, o_ref: np.ndarray, lse_ref: np.ndarray):
    o_gpu = o_gpu.astype(np.float64)
    lse_gpu = lse_gpu.astype(np.float64)
    finite = bool(np.isfinite(o_gpu).all() and np.isfinite(lse_gpu).all())
    e = np.abs(o_gpu - o_ref)
    el = np.abs(lse_gpu - lse_ref)
    where = tuple(int(x) for x in np.unravel_index(int(np.argmax(e)), e.shape)) if e.size else ()
    return dict(finite=finite, max_o=float(e.max()) if e.size else 0.0, mean_o=float(e.mean()) if e.size else 0.0,
                max_lse=float(el.max()) if el.size else 0.0, n=int(e.size),
                p9999_o=float(np.quantile(e, 0.9999)) if e.size else 0.0, argmax_o=where)


def check(st, tag=""):
    say("  %s: max|dO| %.3e at %s, 99.99th pct %.3e, mean|dO| %.3e, max|dLSE| %.3e over %d O elements" %
        (tag, st["max_o"], st.get("argmax_o", ()), st.get("p9999_o", 0.0), st["mean_o"], st["max_lse"], st["n"]))
    assert st["finite"], "%s: NaN/Inf in output" % tag
    assert st["max_o"] <= MAX_ABS_O, "%s: max |dO| %.3e > %.1e" % (tag, st["max_o"], MAX_ABS_O)
    assert st["mean_o"] <= MEAN_ABS_O, "%s: mean |dO| %.3e > %.1e" % (tag, st["mean_o"], MEAN_ABS_O)
    assert st["max_lse"] <= MAX_ABS_LSE, "%s: max |dLSE| %.3e > %.1e" % (tag, st["max_lse"], MAX_ABS_LSE)


def full_parity(q, k, v, causal, scale, tag, variant=None):
    """Whole-tensor comparison (small shapes).  q/k/v are CPU fp16 tensors."""
    o, lse = run(q.cuda(), k.cuda(), v.cuda(), causal, scale, variant)
    O, L = oracle_mod.attn_full(q.numpy(), k.numpy(), v.numpy(), causal, scale)
    st = stats(o.cpu().numpy(), lse.cpu().numpy(), O, L)
    check(st, tag)
    return st


def sample_rows(S: int, rng: np.random.Generator, n_random: int = 96):
    fixed = set(range(min(S, 64)))
    for x in (127, 128, 129, 255, 256, 511, 512, S // 2 - 1, S // 2, S // 2 + 1, S - 1):
        if 0 <= x < S:
            fixed.add(x)
    for x in range(max(0, S - 64), S):
        fixed.add(x)
    fixed.update(int(x) for x in rng.integers(0, S, n_random))
    return sorted(fixed)


def sampled_parity(w: inputs.Workload, q, k, v, o, lse, batches, heads=None, n_random=96, tag=""):
    """Compare sampled (batch, head, row) outputs of a full-size run with the oracle.
    q/k/v/o/lse are GPU tensors of the full workload; the oracle regenerates each sampled batch
    entry on the CPU from its seed and checks that it matches what the GPU holds."""
    rng = np.random.default_rng(w.seed)
    rows = sample_rows(w.S, rng, n_random)
    heads = list(range(w.Hq)) if heads is None else heads
    hs = np.repeat(np.array(heads, dtype=np.int32), len(rows))
    rs = np.tile(np.array(rows, dtype=np.int32), len(heads))
    allst = []
    for b in batches:
        qb, kb, vb = inputs.make_batch_cpu(w, b)
        # the seeded regeneration must be the exact data the kernel read
        assert torch.equal(qb, q[b].cpu()) and torch.equal(kb, k[b].cpu()) and torch.equal(vb, v[b].cpu())
        O, L = oracle_mod.attn_rows(qb.numpy(), kb.numpy(), vb.numpy(), hs, rs, w.causal, w.scale)
        rows_t = torch.as_tensor(rs, dtype=torch.long, device=o.device)
        heads_t = torch.as_tensor(hs, dtype=torch.long, device=o.device)
        og = o[b][rows_t, heads_t].cpu().numpy()
        lg = lse[b][heads_t, rows_t].cpu().numpy()
        allst.append(stats(og, lg, O, L))
    n = sum(s["n"] for s in allst)
    worst = max(range(len(allst)), key=lambda x: allst[x]["max_o"])
    si, d = allst[worst]["argmax_o"] if allst[worst]["argmax_o"] else (0, 0)
    st = dict(finite=all(s["finite"] for s in allst), max_o=max(s["max_o"] for s in allst),
              mean_o=sum(s["mean_o"] * s["n"] for s in allst) / n, max_lse=max(s["max_lse"] for s in allst), n=n,
              p9999_o=max(s["p9999_o"] for s in allst),  # the largest per-batch 99.99th percentile
              argmax_o=(batches[worst], int(rs[si]), int(hs[si]), int(d)))  # (b, row, head, d)
    check(st, tag)
    return st


def slice_parity(w: inputs.Workload, q, k, v, o, lse, b: int, h: int, tag=""):
    """Every query row of head h of batch entry b of a full-size run against the oracle (the oracle
    regenerates the batch entry on the CPU from its seed and checks that it is what the GPU read)."""
    qb, kb, vb = inputs.make_batch_cpu(w, b)
    assert torch.equal(qb, q[b].cpu()) and torch.equal(kb, k[b].cpu()) and torch.equal(vb, v[b].cpu())
    rs = np.arange(w.S, dtype=np.int32)
    hs = np.full(w.S, h, dtype=np.int32)
    O, L = oracle_mod.attn_rows(qb.numpy(), kb.numpy(), vb.numpy(), hs, rs, w.causal, w.scale)
    st = stats(o[b, :, h].cpu().numpy(), lse[b, h].cpu().numpy(), O, L)
    check(st, tag)
    return st


def sampled_parity_shape(w: inputs.VariantShape, q, k, v, o, lse, batches, heads, n_random=64, tag=""):
    """sampled_parity for a variant shape (Sq query rows against Sk keys): sampled (batch, head, row)
    outputs of a full-size run against the oracle, which regenerates each batch entry on the CPU from its
    seed and checks that it is what the GPU read."""
    rng = np.random.default_rng(w.seed)
    rows = sample_rows(w.Sq, rng, n_random)
    hs = np.repeat(np.array(heads, dtype=np.int32), len(rows))
    rs = np.tile(np.array(rows, dtype=np.int32), len(heads))
    allst = []
    for b in batches:
        qb, kb, vb = inputs.make_variant_batch_cpu(w, b)
        assert torch.equal(qb, q[b].cpu()) and torch.equal(kb, k[b].cpu()) and torch.equal(vb, v[b].cpu())
        O, L = oracle_mod.attn_rows(qb.numpy(), kb.numpy(), vb.numpy(), hs, rs, w.causal, w.scale)
        rows_t = torch.as_tensor(rs, dtype=torch.long, device=o.device)
        heads_t = torch.as_tensor(hs, dtype=torch.long, device=o.device)
        allst.append(stats(o[b][rows_t, heads_t].cpu().numpy(), lse[b][heads_t, rows_t].cpu().numpy(), O, L))
    n = sum(s["n"] for s in allst)
    worst = max(range(len(allst)), key=lambda x: allst[x]["max_o"])
    si, d = allst[worst]["argmax_o"] if allst[worst]["argmax_o"] else (0, 0)
    st = dict(finite=all(s["finite"] for s in allst), max_o=max(s["max_o"] for s in allst),
              mean_o=sum(s["mean_o"] * s["n"] for s in allst) / n, max_lse=max(s["max_lse"] for s in allst), n=n,
              p9999_o=max(s["p9999_o"] for s in allst),  # the largest per-batch 99.99th percentile
              argmax_o=(batches[worst], int(rs[si]), int(hs[si]), int(d)))  # (b, row, head, d)
    check(st, tag)
    return st


def batch_entries_parity(w: inputs.Workload, q, k, v, o, lse, batches, tag=""):
    """Every output (all rows, heads and d) of the given batch entries of a full-size run against the
    oracle, the bar applied to all of them together.  The oracle regenerates each batch entry on the CPU
    from its seed and checks that it is what the GPU read."""
    allst = []
    for b in batches:
        qb, kb, vb = inputs.make_batch_cpu(w, b)
        assert torch.equal(qb, q[b].cpu()) and torch.equal(kb, k[b].cpu()) and torch.equal(vb, v[b].cpu())
        O, L = oracle_mod.attn_full(qb.numpy()[None], kb.numpy()[None], vb.numpy()[None], w.causal, w.scale)
        allst.append(stats(o[b:b + 1].cpu().numpy(), lse[b:b + 1].cpu().numpy(), O, L))
        say("  batch entry %d: max |dO| %.3e, max |dLSE| %.3e" % (b, allst[-1]["max_o"], allst[-1]["max_lse"]))
    n = sum(s["n"] for s in allst)
    worst = max(range(len(allst)), key=lambda x: allst[x]["max_o"])
    st = dict(finite=all(s["finite"] for s in allst), max_o=max(s["max_o"] for s in allst),
              mean_o=sum(s["mean_o"] * s["n"] for s in allst) / n, max_lse=max(s["max_lse"] for s in allst), n=n,
              p9999_o=max(s["p9999_o"] for s in allst),  # the largest per-batch 99.99th percentile
              argmax_o=(batches[worst],) + allst[worst]["argmax_o"][1:])  # (b, row, head, d)
    check(st, tag)
    return st


def whole_output_sane(o, lse):
    """Properties that hold at any size: everything finite, |O| bounded by max |V|."""
    assert bool(torch.isfinite(o).all().item()), "non-finite O"
    assert bool(torch.isfinite(lse).all().item()), "non-finite LSE"
