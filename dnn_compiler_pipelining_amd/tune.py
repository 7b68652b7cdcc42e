"""Schedule-space search for libattn.

PipeThreader schedules an operator by searching the space of task orders on
the hardware's units under a resource check, with measured feedback (page
"PipeThreader: Software-Defined Pipelining ... (OSDI 2025)" summary, section
"核心方法").  This module does that for libattn's space of kernel variants
(csrc/variant.h): tile schedule (which also fixes the query rows per wave, 32
or 64) x fragment-prefetch depth x placement of the softmax parts among the
MFMAs (64-row and overlap schedules) x keys per K/V tile (32, 64 or 128; the serial
schedules) (compile time) x query heads per workgroup of the 64-row schedule (4,
2 or 1: 64, 128 or 256 query rows of each) and two workgroup-order switches (run
time).  Variants
with the same tile size compute the same bits; the tile size changes the
rounding order of the online softmax, and every instance is checked against
the oracle, so the search only trades speed.

    python -m dnn_compiler_pipelining_amd.tune --check
        validity of every compiled variant from the code-object metadata (CPU)
    python -m dnn_compiler_pipelining_amd.tune --search OUT_DIR [--workload NAME ...]
        greedy coordinate search with measured feedback per workload (GPU);
        writes OUT_DIR/schedule_search.json
    python -m dnn_compiler_pipelining_amd.tune --emit SEARCH_JSON
        turns a search record into csrc/tuned_table.h and profiles/schedule_search.json (CPU)
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
TABLE = os.path.join(PKG, "csrc", "tuned_table.h")
PROFILE = os.path.join(ROOT, "profiles", "schedule_search.json")

SCHEDULES = ("serial", "overlap", "pingpong", "serial4", "wide", "serial4_16")  # Schedule enum order in csrc/variant.h
PLACES = ("even", "front", "early")  # Place enum order in csrc/variant.h; wide and overlap, the others even only


BNS = (32, 64, 128)  # keys per K/V tile; 32 and 128 for the serial schedules at head dimension 128


def workgroups_per_cu(schedule: str, hd: int, bn: int = 64) -> int:
    """serial4 runs two 4-wave workgroups per CU, except at head dimension 256 or with 128-key tiles (one);
    wide one of 4 waves; the others one of 8 waves."""
    return 2 if schedule.startswith("serial4") and hd <= 128 and bn <= 64 else 1


def waves_per_simd(schedule: str, hd: int, bn: int = 64) -> int:
    """wide (64 query rows per wave) and serial4 at one workgroup per CU run one wave per SIMD; the others
    two."""
    if schedule == "wide":
        return 1
    if schedule.startswith("serial4"):
        return workgroups_per_cu(schedule, hd, bn)
    return 2


def schedule_has(schedule: str, field: str) -> bool:
    """Whether a schedule has more than one value of a variant field: the placement is the wide and overlap
    schedules', the tile size the serial schedules', the heads per workgroup the wide schedule's."""
    if field == "place":
        return schedule in ("wide", "overlap")
    if field == "hpw":
        return schedule == "wide"
    if field == "bn":
        return schedule in ("serial", "serial4")
    return True


RINGS = (2, 4)
SWITCHES = (0, 1)
HPWS = (4, 2, 1)  # query heads per workgroup of the wide schedule; 0 = the largest that divides the GQA ratio
SEED = {"ring": 4, "xcd": 1, "lpt": 1, "place": "even", "bn": 64, "hpw": 0}  # each schedule's search starts here
# A change is kept when it is this much faster.  The median of five timed batches repeats to about
# 0.2% on one box (repeated same-box pairs of the serial and overlap schedules on the 70B-shaped
# B = 16 S = 8192 problem differed by 0.3-1.1%, always in the same direction).
KEEP_GAIN = 0.005

# resource budget of one variant: the SIMD's 512 VGPRs + AGPRs per lane shared by its waves, and 160 KiB of
# LDS shared by the workgroups of a CU
REGISTER_FILE = 512
MAX_LDS = 160 * 1024


def loop_scratch(text: str, symbol: str) -> int:
    """Scratch (spill) instructions inside the loops of one kernel of a device asm file: the instructions of
    every basic block the compiler annotates as a loop header or as inside a loop."""
    start = text.index("\n" + symbol + ":")
    end = text.index(".Lfunc_end", start)
    n, in_loop = 0, False
    for line in text[start:end].split("\n"):
        s = line.strip()
        if re.match(r"^\.LBB\d+_\d+:", s):
            in_loop = "Loop Header" in s or "in Loop:" in s
            continue
        if in_loop and s.startswith("scratch_"):
            n += 1
    return n


def kernel_resources(asm_path: str):
    """{(schedule, ring, hd, place, bn): {vgpr, agpr, vgpr_spill, scratch, lds, loop_scratch}} from the AMDGPU
    metadata of a device asm file and the annotated loop structure of its code.

    The split-KV instances (attn_fwd_decode) appear under the schedule name "serial4-split".  On gfx950
    `vgpr` (.vgpr_count) is the unified register count, AGPRs included; `agpr` is the AGPR part of it."""
    text = open(asm_path).read()
    meta = text[text.index("amdhsa.kernels:"):]
    out = {}
    for block in re.split(r"\n  - ", meta)[1:]:
        m = re.search(r"\.name:\s+\S*attn_fwd_kernelILi(\d)ELi(\d)ELi(\d+)ELb([01])E(?:Li(\d+)E)?(?:Li(\d)E)?",
                      block)
        mw = re.search(r"\.name:\s+\S*attn_wide_kernelILi(\d)ELi(\d)E", block)
        ms = re.search(r"\.name:\s+\S*attn_s16_kernelILi(\d)E", block)
        if not m and not mw and not ms:
            continue

        def num(key):
            mm = re.search(r"\." + key + r":\s+(\d+)", block)
            return int(mm.group(1)) if mm else 0

        if mw:  # the wide kernel: head dimension 128, template arguments = prefetch depth, placement
            key = ("wide", int(mw.group(1)), 128, PLACES[int(mw.group(2))], 64)
        elif ms:  # the 16 x 16 x 32 serial4 kernel: head dimension 128, 64-key tiles; template argument = depth
            key = ("serial4_16", int(ms.group(1)), 128, "even", 64)
        else:
            key = (SCHEDULES[int(m.group(1))] + ("-split" if m.group(4) == "1" else ""), int(m.group(2)),
                   int(m.group(3)), PLACES[int(m.group(6) or 0)], int(m.group(5) or 64))
        sym = re.search(r"\.name:\s+(\S+)", block).group(1)
        out[key] = dict(
            vgpr=num("vgpr_count"), agpr=num("agpr_count"), vgpr_spill=num("vgpr_spill_count"),
            scratch=num("private_segment_fixed_size"), lds=num("group_segment_fixed_size"),
            loop_scratch=loop_scratch(text, sym))
    return out


def check_valid(res: dict, schedule: str = "serial", hd: int = 128, bn: int = 64) -> tuple[bool, str]:
    """A variant is valid when its waves per SIMD fit the register file, no spill traffic runs inside its tile
    loop (spill code executed once per workgroup, in the prologue, the epilogue or the last tile's rare
    redo, is allowed: `wide` at 64 query rows per wave has a little), and the LDS of the workgroups that share
    a CU fits it.  Without the loop structure (res without loop_scratch) any spill is invalid."""
    max_regs = REGISTER_FILE // waves_per_simd(schedule, hd, bn)
    if res["vgpr"] > max_regs:
        return False, "%d VGPRs (AGPRs included) > %d" % (res["vgpr"], max_regs)
    if res.get("loop_scratch", res["vgpr_spill"] or res["scratch"]):
        return False, "spills %d VGPRs / %d B scratch, %s scratch instructions in the tile loop" % (
            res["vgpr_spill"], res["scratch"], res.get("loop_scratch", "?"))
    wg = workgroups_per_cu(schedule, hd, bn)
    if wg * res["lds"] > MAX_LDS:
        return False, "%d x %d B LDS > %d" % (wg, res["lds"], MAX_LDS)
    if res["vgpr_spill"]:
        return True, "ok (%d VGPRs spilled outside the tile loop)" % res["vgpr_spill"]
    return True, "ok"


def valid_variants(asm_paths=None):
    """{(schedule, ring, hd, place, bn): (valid, reason, resources)} for the current sources (device assembly
    of every attention kernel source, or the given files)."""
    from dnn_compiler_pipelining_amd import build

    if asm_paths is None:
        pairs = []
        for src in build.ATTN_SOURCES:
            if not src.endswith(".hip"):
                continue
            fd, path = tempfile.mkstemp(suffix=".s")
            os.close(fd)
            pairs.append((path, src))
        build.device_asm_many(pairs)
        asm_paths = [path for path, _ in pairs]
    elif isinstance(asm_paths, str):
        asm_paths = [asm_paths]
    res = {}
    for path in asm_paths:
        res.update(kernel_resources(path))
    return {k: check_valid(v, k[0], k[2], k[4]) + (v,) for k, v in res.items()}


def variant_key(pt: dict, hd: int) -> tuple:
    """The valid_variants() key of a search point."""
    return (pt["schedule"], pt["ring"], hd, pt.get("place", "even"), pt.get("bn", 64))


# ------------------------------------------------------------------ search (GPU)

def _time(fn, reps: int) -> float:
    import torch

    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def measure(w, point: dict, q, k, v, o, lse) -> float:
    """TFLOP/s of one variant on one workload (median of five timed batches)."""
    from dnn_compiler_pipelining_amd import binding

    reps = max(2, min(50, int(0.15 / max(w.flops / 1e15, 1e-6))))  # about 0.15 s per batch at 1 PFLOP/s
    ms = sorted(_time(lambda: binding.forward(q, k, v, w.causal, w.scale, o, lse, variant=point), reps)
                for _ in range(5))[2]
    return w.flops / ms / 1e9


def greedy_search(rate, is_valid):
    """Greedy coordinate search per schedule: from the schedule's seed (SEED), change one of its fields at a
    time, keep a change only when it is more than KEEP_GAIN faster, repeat until nothing improves; the best
    of the schedules' optima wins.  Searching each schedule on its own keeps the fields that only some
    schedules have (placement, tile size) in the search whichever schedule is fastest.  `rate(point)` is the
    measured TFLOP/s of a point, `is_valid(point)` the resource check; returns (best point, its rate)."""
    fields = [("ring", RINGS), ("xcd", SWITCHES), ("lpt", SWITCHES), ("place", PLACES), ("bn", BNS),
              ("hpw", HPWS)]
    best, best_rate = None, 0.0
    for sched in SCHEDULES:
        cur = dict(SEED, schedule=sched)
        if not is_valid(cur):
            continue
        cur_rate = rate(cur)
        improved = True
        while improved:
            improved = False
            for field, values in fields:
                if not schedule_has(sched, field):
                    continue
                for val in values:
                    if val == cur[field]:
                        continue
                    cand = dict(cur, **{field: val})
                    if not is_valid(cand):
                        continue
                    r = rate(cand)
                    if r > cur_rate * (1.0 + KEEP_GAIN):
                        cur, cur_rate, improved = cand, r, True
        if cur_rate > best_rate:
            best, best_rate = cur, cur_rate
    return best, best_rate


def search_workload(w, valid, log=print):
    """greedy_search on one workload, every point timed on the GPU (measure)."""
    from dnn_compiler_pipelining_amd import inputs

    q, k, v = inputs.make_inputs(w, "cuda")
    import torch

    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.S), dtype=torch.float32, device=q.device)
    seen = {}

    g = w.Hq // w.Hkv
    auto_hpw = 4 if g % 4 == 0 else 2 if g % 2 == 0 else 1

    def rate(pt):
        # hpw 0 runs the largest divisor of the GQA ratio: the same launch as that value, timed once
        hpw = pt["hpw"] or (auto_hpw if pt["schedule"] == "wide" else 0)
        key = (pt["schedule"], pt["ring"], pt["xcd"], pt["lpt"], pt["place"], pt["bn"], hpw)
        if key not in seen:
            seen[key] = measure(w, pt, q, k, v, o, lse)
            log("  %-26s %-9s ring %d xcd %d lpt %d place %-5s bn %3d hpw %d: %7.1f TFLOP/s"
                % (w.name, *key, seen[key]))
        return seen[key]

    best, best_rate = greedy_search(rate, lambda pt: valid.get(variant_key(pt, w.D), (False,))[0])
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    return {"workload": w.name, "B": w.B, "Sq": w.S, "Sk": w.S, "Hq": w.Hq, "Hkv": w.Hkv, "best": best,
            "best_tflops": round(best_rate, 1),
            "measured": [{"schedule": s, "ring": r, "xcd": x, "lpt": l, "place": pl, "bn": bn, "hpw": hp,
                          "tflops": round(t, 1)} for (s, r, x, l, pl, bn, hp), t in seen.items()]}


def search(out_dir: str, names=None):
    from dnn_compiler_pipelining_amd import inputs

    valid = valid_variants()
    for (s, r, hd, pl, bn), (ok, why, _) in sorted(valid.items()):
        print("variant %-13s ring %d hd %3d place %-5s bn %3d: %s" % (s, r, hd, pl, bn, why), flush=True)
    rec = {"valid": {"%s/%d/%d/%s/%d" % k: dict(ok=v[0], reason=v[1], **v[2]) for k, v in valid.items()},
           "rule": "greedy coordinate search per schedule from %s over the fields the schedule has; a change is "
                   "kept when > %.1f%% faster (median of five timed batches); the fastest schedule optimum wins"
                   % (json.dumps(SEED), 100 * KEEP_GAIN),
           "results": []}
    for w in inputs.WORKLOADS:
        if names and w.name not in names:
            continue
        print("search %s" % w.name, flush=True)
        rec["results"].append(search_workload(w, valid, log=lambda *a: print(*a, flush=True)))
    os.makedirs(out_dir, exist_ok=True)
    path = os.path.join(out_dir, "schedule_search.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print("wrote", path)
    return rec


# ------------------------------------------------------------------ emit the table (CPU)

def emit(search_json: str, table: str = TABLE, profile: str | None = PROFILE):
    rec = json.load(open(search_json))
    enum = {name: "SCHEDULE_" + name.upper() for name in SCHEDULES}
    penum = {name: "PLACE_" + name.upper() for name in PLACES}
    lines = ["// tuned_table.h -- generated by `python -m dnn_compiler_pipelining_amd.tune --emit`",
             "// from the measured schedule search (profiles/schedule_search.json); do not edit by hand.",
             "#pragma once", "static const TunedEntry kTuned[] = {"]
    for r in rec["results"]:
        b = r["best"]
        lines.append("    {%d, %d, %d, %d, %d, {%s, %d, %d, %d, %s, %d, %d}, %.1f},  // %s" % (
            r["B"], r["Sq"], r["Sk"], r["Hq"], r["Hkv"], enum[b["schedule"]], b["ring"], b["xcd"], b["lpt"],
            penum[b.get("place", "even")], b.get("bn", 64), b.get("hpw", 0), r["best_tflops"], r["workload"]))
    lines += ["};", "static const int kTunedCount = sizeof(kTuned) / sizeof(kTuned[0]);", ""]
    with open(table, "w") as f:
        f.write("\n".join(lines))
    rec["commands"] = ["python -m dnn_compiler_pipelining_amd.tune --search <out dir>   (on the GPU)",
                       "python -m dnn_compiler_pipelining_amd.tune --emit <out dir>/schedule_search.json"]
    if profile:
        os.makedirs(os.path.dirname(profile), exist_ok=True)
        with open(profile, "w") as f:
            json.dump(rec, f, indent=1)
    print("\n".join(lines))


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--check", action="store_true")
    ap.add_argument("--search", metavar="OUT_DIR")
    ap.add_argument("--workload", action="append")
    ap.add_argument("--emit", metavar="SEARCH_JSON")
    args = ap.parse_args(argv)
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    if args.check:
        for (s, r, hd, pl, bn), (ok, why, res) in sorted(valid_variants().items()):
            print("%-13s ring %d hd %3d place %-5s bn %3d: %-5s %s  %s" % (s, r, hd, pl, bn, ok, why, res))
    if args.search:
        search(args.search, args.workload)
    if args.emit:
        emit(args.emit)
    return 0


if __name__ == "__main__":
    sys.exit(main())
