"""CPU tests of the variant space and its selection (csrc/variant.h, dnn_compiler_pipelining_amd/tune.py)."""
import json
import os
import shutil
import subprocess

import pytest

from dnn_compiler_pipelining_amd import tune

CSRC = os.path.join(tune.PKG, "csrc")


def test_every_compiled_variant_is_valid():
    """Every compiled instance is in the space and passes the check, except the 8-wave serial schedule with
    128-key tiles: at two waves per SIMD its S^T (64 registers) and P^T (32) for 128 keys push it past 256
    registers and it spills inside the tile loop, so the check takes it out of the search."""
    vs = tune.valid_variants()
    rejected = {("serial", r, 128, "even", 128) for r in tune.RINGS}
    assert set(vs) == ({(s, r, 128, "even", 64) for s in tune.SCHEDULES if s not in ("wide", "serial4_16")
                        for r in tune.RINGS} |
                       {(s, r, 128, pl, 64) for s in ("wide", "overlap") for r in tune.RINGS for pl in tune.PLACES} |
                       {("serial4_16", r, 128, "even", 64) for r in tune.RINGS} |
                       {(s, r, 128, "even", bn) for s in ("serial", "serial4") for r in tune.RINGS
                        for bn in (32, 128)} |
                       {(s, r, 64, "even", 64) for s in ("serial", "serial4") for r in tune.RINGS} |
                       {("serial4", r, 256, "even", 64) for r in tune.RINGS} |
                       {("serial4-split", r, hd, "even", 64) for r in tune.RINGS for hd in (64, 128, 256)})
    for key, (ok, why, res) in vs.items():
        assert ok == (key not in rejected), (key, why, res)
        if not ok:
            assert "tile loop" in why, (key, why)
        assert res["lds"] > 0 and res["vgpr"] > 0


@pytest.mark.parametrize("res,reason", [
    (dict(vgpr=257, agpr=0, vgpr_spill=0, scratch=0, lds=1024), "VGPRs"),
    (dict(vgpr=264, agpr=64, vgpr_spill=0, scratch=0, lds=1024), "VGPRs"),
    (dict(vgpr=200, agpr=0, vgpr_spill=3, scratch=12, lds=1024), "spills"),
    (dict(vgpr=200, agpr=0, vgpr_spill=0, scratch=16, lds=1024), "spills"),
    (dict(vgpr=200, agpr=0, vgpr_spill=3, scratch=12, lds=1024, loop_scratch=2), "tile loop"),
    (dict(vgpr=200, agpr=0, vgpr_spill=0, scratch=0, lds=160 * 1024 + 16), "LDS"),
])
def test_check_valid_rejects_over_budget(res, reason):
    ok, why = tune.check_valid(res)
    assert not ok and reason in why


def test_check_valid_allows_spills_outside_the_tile_loop():
    res = dict(vgpr=512, agpr=256, vgpr_spill=28, scratch=112, lds=135168, loop_scratch=0)
    ok, why = tune.check_valid(res, "wide")
    assert ok and "outside the tile loop" in why
    assert not tune.check_valid(dict(res, loop_scratch=1), "wide")[0]
    assert not tune.check_valid(res, "serial")[0]  # 512 registers are one wave per SIMD


def test_loop_scratch_reads_the_loop_annotations():
    asm = "\n".join(["", "k:", "  scratch_load_dword v0, off, off", ".LBB0_1:  ; =>This Inner Loop Header: Depth=1",
                      "  v_add_f32 v1, v1, v1", "  scratch_store_dword off, v1, off", ".LBB0_2:  ;   in Loop: Header=BB0_1 Depth=1",
                      "  scratch_load_dword v2, off, off", ".LBB0_3:", "  scratch_load_dword v3, off, off", ".Lfunc_end0:"])
    assert tune.loop_scratch(asm, "k") == 2


def test_check_valid_counts_two_workgroups_per_cu_for_serial4():
    res = dict(vgpr=180, agpr=0, vgpr_spill=0, scratch=0, lds=84992)
    assert tune.check_valid(res, "serial")[0]
    ok, why = tune.check_valid(res, "serial4")
    assert not ok and "LDS" in why
    # head dimension 256: one workgroup per CU, one wave per SIMD with the whole register file
    big = dict(vgpr=456, agpr=200, vgpr_spill=0, scratch=0, lds=133120)
    assert tune.check_valid(big, "serial4", 256)[0]
    assert not tune.check_valid(big, "serial4", 128)[0]


def test_check_valid_serial4_with_128_key_tiles_runs_one_workgroup_per_cu():
    # 128-key tiles: 135168 B of LDS, so one SERIAL4 workgroup per CU and the whole register file per wave
    res = dict(vgpr=401, agpr=145, vgpr_spill=0, scratch=0, lds=135168, loop_scratch=0)
    assert tune.check_valid(res, "serial4", 128, 128)[0]
    assert not tune.check_valid(res, "serial4", 128, 64)[0]
    assert tune.workgroups_per_cu("serial4", 128, 32) == 2 and tune.workgroups_per_cu("serial4", 128, 128) == 1


def test_greedy_search_covers_each_schedules_own_fields():
    """A synthetic rate table: the wide schedule is fastest, but the serial schedules are still searched
    over their tile sizes and the wide and overlap ones over their placements; invalid points are never
    timed."""
    def rate_of(pt):
        base = {"serial": 100.0, "overlap": 110.0, "pingpong": 105.0, "serial4": 120.0, "wide": 200.0,
                "serial4_16": 118.0}[pt["schedule"]]
        base *= {32: 1.1, 64: 1.0, 128: 0.9}[pt["bn"]] if pt["schedule"] in ("serial", "serial4") else 1.0
        base *= {"even": 1.0, "front": 1.02, "early": 1.05}[pt["place"]] if pt["schedule"] in ("wide", "overlap") else 1.0
        return base * (1.01 if pt["ring"] == 2 else 1.0)

    timed = []

    def rate(pt):
        timed.append(dict(pt))
        return rate_of(pt)

    def is_valid(pt):
        return not (pt["schedule"] == "serial" and pt["bn"] == 128)

    best, r = tune.greedy_search(rate, is_valid)
    assert best == {"schedule": "wide", "ring": 2, "xcd": 1, "lpt": 1, "place": "early", "bn": 64, "hpw": 0}
    assert abs(r - 200.0 * 1.05 * 1.01) < 1e-9
    assert all(is_valid(pt) for pt in timed)
    for sched in ("serial", "serial4"):
        assert {pt["bn"] for pt in timed if pt["schedule"] == sched} == ({32, 64} if sched == "serial" else {32, 64, 128})
        assert {pt["place"] for pt in timed if pt["schedule"] == sched} == {"even"}
    for sched in ("wide", "overlap"):
        assert {pt["place"] for pt in timed if pt["schedule"] == sched} == set(tune.PLACES)
    assert {pt["place"] for pt in timed if pt["schedule"] == "pingpong"} == {"even"}
    assert {pt["bn"] for pt in timed if pt["schedule"] != "serial" and pt["schedule"] != "serial4"} == {64}
    assert {pt["hpw"] for pt in timed if pt["schedule"] == "wide"} == {0, 4, 2, 1}
    assert {pt["hpw"] for pt in timed if pt["schedule"] != "wide"} == {0}


LOOKUP_MAIN = r'''
#include <cstdio>
#include "variant.h"
int main(int argc, char** argv) {
  int B, Sq, Sk, Hq, Hkv;
  while (std::scanf("%d %d %d %d %d", &B, &Sq, &Sk, &Hq, &Hkv) == 5) {
    libattn::Variant v = libattn::tuned_variant(B, Sq, Sk, Hq, Hkv);
    std::printf("%d %d %d %d %d %d %d %d\n", v.schedule, v.ring, v.xcd, v.lpt, v.place, v.bn, v.hpw,
                libattn::variant_valid(v) ? 1 : 0);
  }
  return 0;
}
'''


def lookup(tmp_path, table_dir, shapes):
    # variant.h includes "tuned_table.h" from its own directory, so it is compiled next to the table under test
    if os.path.abspath(str(table_dir)) != os.path.abspath(CSRC):
        shutil.copy(os.path.join(CSRC, "variant.h"), str(table_dir))
    src = tmp_path / "lookup.cpp"
    src.write_text(LOOKUP_MAIN)
    exe = tmp_path / "lookup"
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", str(table_dir), str(src), "-o", str(exe)], check=True)
    inp = "\n".join(" ".join(str(x) for x in s) for s in shapes) + "\n"
    out = subprocess.run([str(exe)], input=inp, capture_output=True, text=True, check=True).stdout.split("\n")
    return [tuple(int(x) for x in line.split()) for line in out if line.strip()]


def test_committed_table_picks_its_own_entries(tmp_path):
    text = open(os.path.join(CSRC, "tuned_table.h")).read()
    import re
    from dnn_compiler_pipelining_amd import binding

    enum = {"SCHEDULE_" + name.upper(): value for name, value in binding.SCHEDULES.items()}
    penum = {"PLACE_" + name.upper(): value for name, value in binding.PLACES.items()}
    rows = re.findall(r"\{(\d+), (\d+), (\d+), (\d+), (\d+), \{(SCHEDULE_\w+), (\d), (\d), (\d), (PLACE_\w+), "
                      r"(\d+), (\d)\}", text)
    assert rows
    got = lookup(tmp_path, CSRC, [r[:5] for r in rows])
    for r, g in zip(rows, got):
        assert g == (enum[r[5]], int(r[6]), int(r[7]), int(r[8]), penum[r[9]], int(r[10]), int(r[11]), 1), (r, g)


def test_emit_and_nearest_shape(tmp_path):
    """A search record becomes a table; a shape takes the variant of the nearest measured shape."""
    rec = {"results": [
        {"workload": "small", "B": 1, "Sq": 512, "Sk": 512, "Hq": 32, "Hkv": 8, "best_tflops": 90.0,
         "best": {"schedule": "overlap", "ring": 2, "xcd": 0, "lpt": 1}},
        {"workload": "big", "B": 64, "Sq": 8192, "Sk": 8192, "Hq": 64, "Hkv": 8, "best_tflops": 990.0,
         "best": {"schedule": "pingpong", "ring": 4, "xcd": 1, "lpt": 0}},
        {"workload": "mid", "B": 64, "Sq": 2048, "Sk": 2048, "Hq": 32, "Hkv": 8, "best_tflops": 850.0,
         "best": {"schedule": "wide", "ring": 4, "xcd": 1, "lpt": 1, "place": "early"}},
        {"workload": "short", "B": 4, "Sq": 256, "Sk": 256, "Hq": 8, "Hkv": 8, "best_tflops": 40.0,
         "best": {"schedule": "serial4", "ring": 2, "xcd": 0, "lpt": 0, "place": "even", "bn": 32}},
        {"workload": "wide2", "B": 2, "Sq": 16384, "Sk": 16384, "Hq": 16, "Hkv": 8, "best_tflops": 900.0,
         "best": {"schedule": "wide", "ring": 4, "xcd": 1, "lpt": 1, "place": "even", "bn": 64, "hpw": 2}},
    ]}
    js = tmp_path / "search.json"
    js.write_text(json.dumps(rec))
    tdir = tmp_path / "tbl"
    tdir.mkdir()
    tune.emit(str(js), table=str(tdir / "tuned_table.h"), profile=None)
    got = lookup(tmp_path, tdir, [(1, 600, 600, 32, 8), (48, 8192, 8192, 64, 8), (1, 2048, 8192, 64, 8),
                                  (64, 2000, 2000, 32, 8), (4, 200, 200, 8, 8), (2, 16000, 16000, 16, 8)])
    assert got[0] == (1, 2, 0, 1, 0, 64, 0, 1)
    assert got[1] == (2, 4, 1, 0, 0, 64, 0, 1)
    assert got[2] in ((1, 2, 0, 1, 0, 64, 0, 1), (2, 4, 1, 0, 0, 64, 0, 1))
    assert got[3] == (4, 4, 1, 1, 2, 64, 0, 1)
    assert got[4] == (3, 2, 0, 0, 0, 32, 0, 1)
    assert got[5] == (4, 4, 1, 1, 0, 64, 2, 1)


def test_committed_table_is_what_the_committed_search_emits(tmp_path):
    """tuned_table.h is generated: emitting the committed search record gives the committed file byte for byte,
    so the table the library compiles in is the one the recorded measurements chose."""
    from dnn_compiler_pipelining_amd import tune

    out = tmp_path / "tuned_table.h"
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    tune.emit(os.path.join(root, "profiles", "schedule_search.json"), table=str(out), profile=None)
    assert out.read_text() == open(os.path.join(CSRC, "tuned_table.h")).read()
