"""Build libattn.so (gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

WIDE_SOURCES = [os.path.join(CSRC, "attn_wide_%s.hip" % p) for p in ("even", "front", "early")]
ATTN_SOURCES = [os.path.join(CSRC, "attn_fwd.hip"), *WIDE_SOURCES, os.path.join(CSRC, "attn_s16.hip"),
                os.path.join(CSRC, "attn_api.cpp"), os.path.join(CSRC, "attn_static_ws.hip")]
GEMM_SOURCES = [os.path.join(CSRC, "gemm_fwd.hip"), os.path.join(CSRC, "gemm_api.cpp")]
# measurement aid (attn_mfma_ceiling), outside the attention and GEMM paths
PROBE_SOURCES = [os.path.join(CSRC, "mfma_ceiling.hip")]
SOURCES = ATTN_SOURCES + GEMM_SOURCES + PROBE_SOURCES

# Packed fp32 VALU forms are switched off for all device code.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I" + INCLUDE, "-I" + CSRC]


def build(out: str = LIB, extra_flags=()) -> str:
    """Compile libattn.so (always recompiles): each source to an object in parallel, then one link.  Returns
    the library path."""
    tmpdir = tempfile.mkdtemp(prefix="libattn_build_")
    try:
        procs = []
        for src in SOURCES:
            obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
            cmd = [HIPCC, *[f for f in HIP_FLAGS if f != "-shared"], *extra_flags, "-c", src, "-o", obj]
            procs.append((cmd, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        for cmd, _, proc in procs:
            _, err = proc.communicate()
            if proc.returncode != 0:
                raise RuntimeError("hipcc failed (%d):\n%s\n%s" % (proc.returncode, " ".join(cmd), err))
        tmp = out + ".tmp%d" % os.getpid()
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[obj for _, obj, _ in procs], "-o", tmp]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("hipcc link failed (%d):\n%s\n%s" % (res.returncode, " ".join(cmd), res.stderr))
        os.replace(tmp, out)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return out


def _asm_cmd(out: str, src: str):
    return [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-S", "--cuda-device-only",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I" + INCLUDE, "-I" + CSRC, src, "-o", out]


def device_asm(out: str, src: str | None = None) -> str:
    """Write the gfx950 assembly of one kernel source (default: the attention kernel), for register, LDS and
    scratch inspection."""
    subprocess.run(_asm_cmd(out, src or ATTN_SOURCES[0]), check=True, capture_output=True)
    return out


def device_asm_many(pairs) -> None:
    """device_asm() for several (out, src) pairs, compiled in parallel."""
    procs = [(src, subprocess.Popen(_asm_cmd(out, src), stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
             for out, src in pairs]
    for src, proc in procs:
        _, err = proc.communicate()
        if proc.returncode != 0:
            raise RuntimeError("hipcc -S failed for %s:\n%s" % (src, err))


if __name__ == "__main__":
    print(build())
