"""CPU tests of the C ABI: the library builds, loads, exports what include/*.h declares,
and rejects invalid arguments before touching the GPU (fake pointers are never dereferenced)."""
import ctypes
import os
import re
import subprocess

import pytest

from dnn_compiler_pipelining_amd import binding as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", n) for n in sorted(os.listdir(os.path.join(ROOT, "include")))
           if n.endswith(".h")]

# Aligned, distinct, never-dereferenced fake device addresses (validation fails before use).
QP, KP, VP, OP, LP = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000


def declared_functions():
    names = set()
    for path in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
        names.update(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b((?:attn|gemm)_\w+)\s*\(", text, flags=re.M))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        from dnn_compiler_pipelining_amd import build
        build.build()
    return L.load()


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(L.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(\w+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_version_and_status_strings(lib):
    assert L.attn_version() >= 10000
    assert L.attn_status_string(L.ATTN_OK) == "ok"
    for code in range(1, 9):
        s = L.attn_status_string(code)
        assert s and s != "unknown status"
    assert L.attn_status_string(99) == "unknown status"


def call(q=QP, k=KP, v=VP, o=OP, lse=LP, B=1, S=64, Hq=8, Hkv=2, D=128, causal=1, scale=0.088):
    return L.attn_fwd(q, k, v, o, lse, B, S, Hq, Hkv, D, causal, scale)


def test_null_pointers(lib):
    assert call(q=0) == L.ATTN_ERR_NULL
    assert call(k=0) == L.ATTN_ERR_NULL
    assert call(v=0) == L.ATTN_ERR_NULL
    assert call(o=0) == L.ATTN_ERR_NULL


@pytest.mark.parametrize("kw", [dict(B=0), dict(S=0), dict(Hq=0), dict(Hkv=0), dict(Hq=6, Hkv=4), dict(causal=2),
                                dict(causal=-1), dict(scale=float("inf")), dict(scale=float("nan")), dict(B=-3)])
def test_bad_shapes(lib, kw):
    assert call(**kw) == L.ATTN_ERR_SHAPE


@pytest.mark.parametrize("D", [96, 512, 127, 32, 1, 192])
def test_unsupported_head_dim(lib, D):
    assert call(D=D) == L.ATTN_ERR_UNSUPPORTED


@pytest.mark.parametrize("which", ["q", "k", "v", "o", "lse"])
def test_misaligned(lib, which):
    kw = {which: {"q": QP, "k": KP, "v": VP, "o": OP, "lse": LP}[which] + 8}
    assert call(**kw) == L.ATTN_ERR_ALIGN


def test_overlap(lib):
    assert call(o=QP) == L.ATTN_ERR_OVERLAP
    assert call(o=KP + 4096) == L.ATTN_ERR_OVERLAP  # o starts inside k
    assert call(o=LP - 4096) == L.ATTN_ERR_OVERLAP  # o runs into lse
    assert call(o=VP, lse=0) == L.ATTN_ERR_OVERLAP
    # lse is written while other workgroups still read q, k and v
    assert call(lse=QP + 256) == L.ATTN_ERR_OVERLAP
    assert call(lse=KP) == L.ATTN_ERR_OVERLAP
    assert call(lse=VP + 1024) == L.ATTN_ERR_OVERLAP


def test_validation_order(lib):
    # a null pointer is reported before a bad shape, a bad shape before an unsupported D
    assert call(q=0, B=0) == L.ATTN_ERR_NULL
    assert call(B=0, D=96) == L.ATTN_ERR_SHAPE
    assert call(D=96, q=QP + 8) == L.ATTN_ERR_UNSUPPORTED


def test_stream_entry_point_validates_too(lib):
    st = L.attn_fwd_stream(QP, KP, VP, OP, LP, 1, 64, 8, 3, 128, 1, 0.1, None)
    assert st == L.ATTN_ERR_SHAPE


def test_binding_fails_loudly_without_library(tmp_path):
    saved = L._lib
    try:
        L._lib = None
        with pytest.raises(FileNotFoundError):
            L.load(str(tmp_path / "missing.so"))
    finally:
        L._lib = saved


def call_ex(**kw):
    a = dict(q=QP, k=KP, v=VP, o=OP, lse=LP, B=1, Sq=64, Sk=64, Hq=8, Hkv=2, D=128, causal=1, scale=0.1, stream=None)
    a.update(kw)
    return L.attn_fwd_ex(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Sq"], a["Sk"], a["Hq"], a["Hkv"], a["D"],
                         a["causal"], a["scale"], a["stream"])


@pytest.mark.parametrize("kw", [dict(Sq=0), dict(Sk=0), dict(Sq=65, Sk=64), dict(Sq=(1 << 30) + 1, Sk=(1 << 30) + 1),
                                dict(Sk=(1 << 30) + 1, causal=0), dict(Hq=9, Hkv=2)], ids=str)
def test_ex_bad_shapes(lib, kw):
    """attn_fwd_ex: causal needs Sq <= Sk; sizes are 1..2^30 (nothing is launched on an error)."""
    assert call_ex(**kw) == L.ATTN_ERR_SHAPE


def test_ex_limits_and_order(lib):
    assert call_ex(D=512) == L.ATTN_ERR_UNSUPPORTED
    # 64 rows of K/V must span less than 4 GiB: Hkv * 128 * 2 * 64 >= 2^32 is refused
    assert call_ex(Hq=262144, Hkv=262144) == L.ATTN_ERR_UNSUPPORTED
    assert call_ex(q=0, Sq=65) == L.ATTN_ERR_NULL
    assert call_ex(Sq=65, D=96) == L.ATTN_ERR_SHAPE
    assert call_ex(o=KP + 4096, Sq=16, Sk=64) == L.ATTN_ERR_OVERLAP


# ---------------------------------------------------------------- gemm_f16 (include/gemm.h)
AP, BP, CP = 0x60000000, 0x70000000, 0x80000000


def gcall(a=AP, b=BP, c=CP, M=300, N=264, K=136, b_layout=0):
    return L.gemm_f16(a, b, c, M, N, K, b_layout, None)


def test_gemm_null_pointers(lib):
    assert gcall(a=0) == L.ATTN_ERR_NULL
    assert gcall(b=0) == L.ATTN_ERR_NULL
    assert gcall(c=0) == L.ATTN_ERR_NULL


def test_gemm_empty_output_launches_nothing(lib):
    # M = 0 or N = 0: nothing to compute, NULL pointers allowed, no GPU touched
    assert gcall(a=0, b=0, c=0, M=0) == L.ATTN_OK
    assert gcall(a=0, b=0, c=0, N=0) == L.ATTN_OK
    assert gcall(M=0, N=0, K=0) == L.ATTN_OK


@pytest.mark.parametrize("kw", [dict(M=-1), dict(N=-8), dict(K=-8), dict(M=(1 << 24) + 1), dict(N=(1 << 24) + 8),
                                dict(K=(1 << 22) + 8), dict(b_layout=2), dict(b_layout=-1)])
def test_gemm_bad_shapes(lib, kw):
    assert gcall(**kw) == L.ATTN_ERR_SHAPE


@pytest.mark.parametrize("kw", [dict(K=130), dict(N=260), dict(K=7, b_layout=1), dict(N=1)])
def test_gemm_unsupported(lib, kw):
    assert gcall(**kw) == L.ATTN_ERR_UNSUPPORTED


def test_gemm_alignment_and_overlap(lib):
    assert gcall(a=AP + 8) == L.ATTN_ERR_ALIGN
    assert gcall(b=BP + 2) == L.ATTN_ERR_ALIGN
    assert gcall(c=CP + 4) == L.ATTN_ERR_ALIGN
    a_bytes = 300 * 136 * 2
    assert gcall(c=AP + 16 * (a_bytes // 32)) == L.ATTN_ERR_OVERLAP  # c starts inside a
    assert gcall(c=BP - 16) == L.ATTN_ERR_OVERLAP                    # c runs into b


def test_gemm_check_order(lib):
    # NULL before shape, shape before unsupported, unsupported before alignment, alignment before overlap
    assert gcall(a=0, M=-1) == L.ATTN_ERR_NULL
    assert gcall(K=130, b_layout=3) == L.ATTN_ERR_SHAPE
    assert gcall(K=130, a=AP + 8) == L.ATTN_ERR_UNSUPPORTED
    assert gcall(a=AP + 8, c=AP) == L.ATTN_ERR_ALIGN


# ---------------------------------------------------------------- attn_fwd_decode (split-KV path)
WSP = 0x90000000


def dcall(ws=WSP, ws_bytes=1 << 30, q=QP, k=KP, v=VP, o=OP, lse=LP, B=2, Sq=1, Sk=8192, Hq=64, Hkv=8, D=128,
          causal=1, scale=0.088):
    return L.attn_fwd_decode(q, k, v, o, lse, B, Sq, Sk, Hq, Hkv, D, causal, scale, ws, ws_bytes, None)


def test_decode_workspace_size(lib):
    # B=2, Sq=1, Sk=8192, 64/8 heads, D=128: 8 packed rows -> one tile per KV group, 16 groups, so the 128 key
    # tiles are cut into 32 splits of 4 tiles (about 512 workgroups); partials are 2*64*1 rows x 32 splits x
    # (128 + 1) floats
    assert L.attn_decode_workspace_size(2, 1, 8192, 64, 8, 128) == 2 * 64 * 32 * 129 * 4
    # a big grid needs no split: one partial per row
    assert L.attn_decode_workspace_size(64, 1024, 8192, 64, 8, 128) == 64 * 64 * 1024 * 129 * 4
    for bad in [(0, 1, 8, 8, 8, 128), (1, 1, 8, 9, 2, 128), (1, 1, 8, 8, 8, 96), (1, 0, 8, 8, 8, 128)]:
        assert L.attn_decode_workspace_size(*bad) == 0


def test_decode_validation(lib):
    need = L.attn_decode_workspace_size(2, 1, 8192, 64, 8, 128)
    assert dcall(q=0) == L.ATTN_ERR_NULL
    assert dcall(Sq=2, Sk=1) == L.ATTN_ERR_SHAPE
    assert dcall(D=96) == L.ATTN_ERR_UNSUPPORTED
    assert dcall(ws=0) == L.ATTN_ERR_WORKSPACE
    assert dcall(ws_bytes=need - 4) == L.ATTN_ERR_WORKSPACE
    assert dcall(ws=WSP + 8) == L.ATTN_ERR_WORKSPACE
    assert dcall(ws=QP) == L.ATTN_ERR_OVERLAP          # workspace over q
    assert dcall(ws=LP - 64) == L.ATTN_ERR_OVERLAP     # workspace running into lse
    assert dcall(q=0, ws=0) == L.ATTN_ERR_NULL          # argument checks come before workspace checks
    assert L.attn_status_string(L.ATTN_ERR_WORKSPACE) != "unknown status"


def test_tuned_variant_reports_a_runnable_variant(lib):
    for B, S, Hq, Hkv, D in ((1, 512, 32, 8, 128), (64, 8192, 64, 8, 128), (2, 100, 8, 2, 64), (1, 33, 4, 4, 256)):
        v = L.attn_tuned_variant(B, S, S, Hq, Hkv, D)
        assert set(v) == {"schedule", "ring", "xcd", "lpt", "place", "bn", "hpw"}
        assert v["hpw"] in (0, 1, 2, 4) and (v["schedule"] == "wide" or v["hpw"] == 0)
        assert v["schedule"] in L.SCHEDULES and v["ring"] in (2, 4) and v["xcd"] in (0, 1) and v["lpt"] in (0, 1)
        assert v["place"] in L.PLACES and (v["schedule"] in ("wide", "overlap") or v["place"] == "even")
        assert v["bn"] == 64 or (v["bn"] in (32, 128) and v["schedule"] in ("serial", "serial4") and D == 128)
        if D != 128:
            assert v["schedule"] in ("serial", "serial4")  # the only schedules D = 64 and 256 run
    out = [ctypes.c_int(0) for _ in range(7)]
    refs = [ctypes.byref(x) for x in out]
    assert lib.attn_tuned_variant(1, 64, 64, 8, 2, 96, *refs) == L.ATTN_ERR_UNSUPPORTED
    assert lib.attn_tuned_variant(1, 64, 64, 6, 4, 128, *refs) == L.ATTN_ERR_SHAPE
    assert lib.attn_tuned_variant(0, 64, 64, 8, 2, 128, *refs) == L.ATTN_ERR_SHAPE
    assert lib.attn_tuned_variant(1, 64, 64, 8, 2, 128, None, *refs[1:]) == L.ATTN_ERR_NULL
    assert lib.attn_device_clock(0, None, refs[0]) == L.ATTN_ERR_NULL


def test_static_decode_validates_before_any_hip_call(lib):
    # invalid arguments keep the split-KV path's codes; sizes past the static workspace are rejected; all
    # before the device is touched
    assert L.attn_fwd_decode_static(QP, KP, VP, OP, LP, 1, 1, 64, 6, 4, 128, 1, 0.06, None) == L.ATTN_ERR_SHAPE
    assert L.attn_fwd_decode_static(0, KP, VP, OP, LP, 1, 1, 64, 8, 4, 128, 1, 0.06, None) == L.ATTN_ERR_NULL
    assert L.attn_fwd_decode_static(QP, KP, VP, OP, LP, 1, 1, 64, 8, 4, 96, 1, 0.06, None) == L.ATTN_ERR_UNSUPPORTED
    assert L.attn_fwd_decode_static(QP + 8, KP, VP, OP, LP, 1, 1, 64, 8, 4, 128, 1, 0.06, None) == L.ATTN_ERR_ALIGN
    assert L.attn_decode_workspace_size(1, 128, 8192, 64, 8, 256) > L.ATTN_STATIC_WORKSPACE_BYTES
    assert L.attn_fwd_decode_static(QP, KP, VP, OP, LP, 1, 128, 8192, 64, 8, 256, 1, 0.06, None) == \
        L.ATTN_ERR_TOO_LARGE
    assert L.attn_fwd_decode_static(0, KP, VP, OP, LP, 1, 128, 8192, 64, 8, 256, 1, 0.06, None) == L.ATTN_ERR_NULL


def test_variant_placements_outside_the_wide_and_overlap_schedules_are_rejected(lib):
    # rejected while choosing the variant, before any HIP call (the pointers are never used)
    def var(schedule, place, D=128, ring=-1):
        return L.attn_fwd_variant(QP, KP, VP, OP, LP, 1, 64, 64, 8, 2, D, 1, 0.088, schedule, ring, -1, -1, place, -1,
                                  -1, None)
    for sched in ("serial", "pingpong", "serial4", "serial4_16"):
        for place in ("front", "early"):
            assert var(L.SCHEDULES[sched], L.PLACES[place]) == L.ATTN_ERR_UNSUPPORTED, (sched, place)
    assert var(L.SCHEDULES["overlap"], 3) == L.ATTN_ERR_UNSUPPORTED
    assert var(L.SCHEDULES["overlap"], L.PLACES["front"], D=64) == L.ATTN_ERR_UNSUPPORTED
    assert var(L.SCHEDULES["wide"], 3) == L.ATTN_ERR_UNSUPPORTED
    assert var(L.SCHEDULES["wide"], L.PLACES["front"], ring=3) == L.ATTN_ERR_UNSUPPORTED
    assert var(L.SCHEDULES["wide"], L.PLACES["early"], D=64) == L.ATTN_ERR_UNSUPPORTED


def test_variant_tile_sizes_outside_the_serial_schedules_are_rejected(lib):
    # 32- and 128-key tiles: SERIAL and SERIAL4 at D = 128 only; rejected before any HIP call
    def var(schedule, bn, D=128):
        return L.attn_fwd_variant(QP, KP, VP, OP, LP, 1, 64, 64, 8, 2, D, 1, 0.088, schedule, -1, -1, -1, -1, bn, -1,
                                  None)
    for sched in ("overlap", "pingpong", "wide", "serial4_16"):
        for bn in (32, 128):
            assert var(L.SCHEDULES[sched], bn) == L.ATTN_ERR_UNSUPPORTED, (sched, bn)
    for sched in ("serial", "serial4"):
        for bn in (0, 16, 48, 96, 256):
            assert var(L.SCHEDULES[sched], bn) == L.ATTN_ERR_UNSUPPORTED, (sched, bn)
        assert var(L.SCHEDULES[sched], 32, D=64) == L.ATTN_ERR_UNSUPPORTED
    assert var(L.SCHEDULES["serial4"], 128, D=256) == L.ATTN_ERR_UNSUPPORTED


def test_variant_heads_per_workgroup_outside_the_wide_schedule_are_rejected(lib):
    # 4, 2 or 1 heads per workgroup (0: the largest dividing Hq / Hkv): the wide schedule only
    def var(schedule, hpw, D=128):
        return L.attn_fwd_variant(QP, KP, VP, OP, LP, 1, 64, 64, 8, 2, D, 1, 0.088, schedule, -1, -1, -1, -1, -1, hpw,
                                  None)
    for sched in ("serial", "overlap", "pingpong", "serial4", "serial4_16"):
        for hpw in (1, 2, 4):
            assert var(L.SCHEDULES[sched], hpw) == L.ATTN_ERR_UNSUPPORTED, (sched, hpw)
    for hpw in (3, 5, 8, 16):
        assert var(L.SCHEDULES["wide"], hpw) == L.ATTN_ERR_UNSUPPORTED, hpw
    assert var(L.SCHEDULES["wide"], 2, D=64) == L.ATTN_ERR_UNSUPPORTED


def test_sixteen_by_sixteen_schedule_runs_head_dimension_128_only(lib):
    def var(schedule, D):
        return L.attn_fwd_variant(QP, KP, VP, OP, LP, 1, 64, 64, 8, 2, D, 1, 0.088, schedule, -1, -1, -1, -1, -1, -1,
                                  None)
    for D in (64, 256):
        assert var(L.SCHEDULES["serial4_16"], D) == L.ATTN_ERR_UNSUPPORTED, D
    assert var(6, 128) == L.ATTN_ERR_UNSUPPORTED  # no such schedule


def test_mfma_ceiling_validates_before_any_hip_call(lib):
    import ctypes
    out = ctypes.c_double(-1.0)
    assert lib.attn_mfma_ceiling(0, None, ctypes.byref(out)) == L.ATTN_ERR_SHAPE
    assert lib.attn_mfma_ceiling(-5, None, ctypes.byref(out)) == L.ATTN_ERR_SHAPE
    assert lib.attn_mfma_ceiling(10000001, None, ctypes.byref(out)) == L.ATTN_ERR_SHAPE
    assert lib.attn_mfma_ceiling(100, None, None) == L.ATTN_ERR_NULL
    for shape in (0, 8, 17, 31, 64):
        assert lib.attn_mfma_ceiling_shape(shape, 100, None, ctypes.byref(out)) == L.ATTN_ERR_UNSUPPORTED, shape
    assert lib.attn_mfma_ceiling_shape(16, 0, None, ctypes.byref(out)) == L.ATTN_ERR_SHAPE
    assert lib.attn_mfma_ceiling_shape(16, 100, None, None) == L.ATTN_ERR_NULL
    assert out.value == -1.0


def header_constants():
    """Every `ATTN_NAME = value` of the enums in include/*.h, and ATTN_STATIC_WORKSPACE_BYTES."""
    consts = {}
    for path in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
        for name, val in re.findall(r"\b(ATTN_[A-Z0-9_]+)\s*=\s*(\d+)", text):
            consts[name] = int(val)
        for name, expr in re.findall(r"#define\s+(ATTN_[A-Z0-9_]+)\s+([^\n]+)", text):
            m = re.search(r"(\d+)\s*<<\s*(\d+)", expr)  # ((size_t)64 << 20)
            if m:
                consts[name] = int(m.group(1)) << int(m.group(2))
    return consts


def test_binding_constants_match_the_header():
    """The binding's status codes, schedule and placement numbers and static workspace size are the
    header's: a drift would pass a different schedule, or misname a status, without any error."""
    h = header_constants()
    codes = {n: v for n, v in h.items() if n == "ATTN_OK" or n.startswith("ATTN_ERR_")}
    assert codes and all(getattr(L, n) == v for n, v in codes.items()), codes
    scheds = {n[len("ATTN_SCHEDULE_"):].lower(): v for n, v in h.items() if n.startswith("ATTN_SCHEDULE_")}
    assert scheds == L.SCHEDULES
    places = {n[len("ATTN_PLACE_"):].lower(): v for n, v in h.items() if n.startswith("ATTN_PLACE_")}
    assert places == L.PLACES
    assert h.get("ATTN_STATIC_WORKSPACE_BYTES") == L.ATTN_STATIC_WORKSPACE_BYTES
