"""Python binding of libattn: argument marshalling only.

The functions carry the names of the C entry points in include/attn.h
(attn_fwd, attn_fwd_stream, attn_fwd_ex, attn_fwd_variant, attn_fwd_decode,
attn_fwd_decode_split, attn_decode_workspace_size,
attn_decode_workspace_size_split, attn_status_string, attn_version) and
include/gemm.h (gemm_f16, gemm_f16_waves) and forward to them through ctypes;
every step of the computation runs in the HIP kernels.  `forward()`, `decode()` and
`matmul()` are conveniences that allocate the outputs (and the decode
workspace) with torch and check the tensors first.  There is no fallback: if libattn.so is missing or fails to
load, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libattn.so")

ATTN_OK = 0
ATTN_ERR_NULL = 1
ATTN_ERR_SHAPE = 2
ATTN_ERR_UNSUPPORTED = 3
ATTN_ERR_ALIGN = 4
ATTN_ERR_HIP = 5
ATTN_ERR_OVERLAP = 6
ATTN_ERR_WORKSPACE = 7
ATTN_ERR_TOO_LARGE = 8
ATTN_STATIC_WORKSPACE_BYTES = 64 << 20  # the library's own split-KV workspace per GPU (attn_fwd_decode_static)

EXPORTS = ("attn_fwd", "attn_fwd_stream", "attn_fwd_ex", "attn_fwd_variant", "attn_fwd_decode",
           "attn_fwd_decode_split", "attn_fwd_decode_static", "attn_decode_workspace_size", "attn_decode_workspace_size_split",
           "attn_status_string", "attn_version", "attn_tuned_variant", "attn_device_clock", "attn_mfma_ceiling", "attn_mfma_ceiling_shape", "gemm_f16",
           "gemm_f16_waves")

# Tile schedules (ATTN_SCHEDULE_* in include/attn.h), by name
SCHEDULES = {"serial": 0, "overlap": 1, "pingpong": 2, "serial4": 3, "wide": 4, "serial4_16": 5}
# Placements of the softmax work in the 64-row schedule (ATTN_PLACE_* in include/attn.h), by name
PLACES = {"even": 0, "front": 1, "early": 2}

GEMM_B_KN = 0  # B stored [K, N]: C = A B
GEMM_B_NK = 1  # B stored [N, K]: C = A B^T

_lock = threading.Lock()
_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int):
        super().__init__("libattn status %d: %s" % (status, attn_status_string(status)))
        self.status = status


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libattn.so.  Raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(path):
                raise FileNotFoundError(
                    "libattn.so not built at %s: run `python -c 'import __graft_entry__ as g; g.build()'`" % path)
            lib = ctypes.CDLL(path)
            vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
            lib.attn_fwd.restype = i
            lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f]
            lib.attn_fwd_stream.restype = i
            lib.attn_fwd_stream.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
            lib.attn_fwd_ex.restype = i
            lib.attn_fwd_ex.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp]
            lib.attn_fwd_variant.restype = i
            lib.attn_fwd_variant.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, i, i, i, i, i, i, vp]
            lib.attn_fwd_decode_split.restype = i
            lib.attn_fwd_decode_split.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp, ctypes.c_size_t,
                                                  vp]
            lib.attn_decode_workspace_size_split.restype = ctypes.c_size_t
            lib.attn_decode_workspace_size_split.argtypes = [i, i, i, i, i, i, i]
            lib.gemm_f16_waves.restype = i
            lib.gemm_f16_waves.argtypes = [vp, vp, vp, i, i, i, i, i, vp]
            lib.attn_fwd_decode.restype = i
            lib.attn_fwd_decode.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp, ctypes.c_size_t, vp]
            lib.attn_fwd_decode_static.restype = i
            lib.attn_fwd_decode_static.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp]
            lib.attn_decode_workspace_size.restype = ctypes.c_size_t
            lib.attn_decode_workspace_size.argtypes = [i, i, i, i, i, i]
            ip = ctypes.POINTER(ctypes.c_int)
            lib.attn_tuned_variant.restype = i
            lib.attn_tuned_variant.argtypes = [i, i, i, i, i, i, ip, ip, ip, ip, ip, ip, ip]
            lib.attn_device_clock.restype = i
            lib.attn_device_clock.argtypes = [i, ip, ip]
            lib.attn_mfma_ceiling.restype = i
            lib.attn_mfma_ceiling.argtypes = [i, vp, ctypes.POINTER(ctypes.c_double)]
            lib.attn_mfma_ceiling_shape.restype = i
            lib.attn_mfma_ceiling_shape.argtypes = [i, i, vp, ctypes.POINTER(ctypes.c_double)]
            lib.attn_status_string.restype = ctypes.c_char_p
            lib.attn_status_string.argtypes = [i]
            lib.attn_version.restype = i
            lib.attn_version.argtypes = []
            lib.gemm_f16.restype = i
            lib.gemm_f16.argtypes = [vp, vp, vp, i, i, i, i, vp]
            _lib = lib
        return _lib


def _ptr(x) -> int:
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    return x.data_ptr()


def attn_fwd(q, k, v, o, lse, B: int, S: int, Hq: int, Hkv: int, D: int, causal: int, scale: float) -> int:
    """C attn_fwd on the null stream.  Tensors or raw device addresses (int); lse may be None."""
    return load().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, S, Hq, Hkv, D, int(causal),
                           float(scale))


def attn_fwd_stream(q, k, v, o, lse, B: int, S: int, Hq: int, Hkv: int, D: int, causal: int, scale: float,
                    stream) -> int:
    """C attn_fwd_stream.  `stream` is a torch.cuda.Stream, a raw hipStream_t (int) or None."""
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else (stream or 0)
    return load().attn_fwd_stream(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, S, Hq, Hkv, D, int(causal),
                                  float(scale), handle)


def attn_fwd_ex(q, k, v, o, lse, B: int, Sq: int, Sk: int, Hq: int, Hkv: int, D: int, causal: int, scale: float,
                stream) -> int:
    """C attn_fwd_ex (Sq query rows, Sk keys).  `stream` as for attn_fwd_stream."""
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else (stream or 0)
    return load().attn_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Sq, Sk, Hq, Hkv, D, int(causal),
                              float(scale), handle)


def attn_fwd_variant(q, k, v, o, lse, B: int, Sq: int, Sk: int, Hq: int, Hkv: int, D: int, causal: int,
                     scale: float, schedule: int, ring: int, xcd: int, lpt: int, place: int, bn: int,
                     hpw: int, stream) -> int:
    """C attn_fwd_variant: attn_fwd_ex with an explicit kernel variant (-1 in a field: the tuned value)."""
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else (stream or 0)
    return load().attn_fwd_variant(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Sq, Sk, Hq, Hkv, D,
                                   int(causal), float(scale), int(schedule), int(ring), int(xcd), int(lpt),
                                   int(place), int(bn), int(hpw), handle)


def attn_fwd_decode_static(q, k, v, o, lse, B: int, Sq: int, Sk: int, Hq: int, Hkv: int, D: int, causal: int,
                           scale: float, stream) -> int:
    """C attn_fwd_decode_static: the split-KV path on the library's own per-GPU workspace (no allocation).
    `stream` as for attn_fwd_stream; the current device must be the stream's."""
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else (stream or 0)
    return load().attn_fwd_decode_static(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Sq, Sk, Hq, Hkv, D,
                                         int(causal), float(scale), handle)


def attn_tuned_variant(B: int, Sq: int, Sk: int, Hq: int, Hkv: int, D: int) -> dict:
    """C attn_tuned_variant: the variant attn_fwd_ex runs for these sizes, as variant_fields() names it."""
    out = [ctypes.c_int(-1) for _ in range(7)]
    st = load().attn_tuned_variant(B, Sq, Sk, Hq, Hkv, D, *[ctypes.byref(x) for x in out])
    if st != ATTN_OK:
        raise AttnError(st)
    names = {v: n for n, v in SCHEDULES.items()}
    places = {v: n for n, v in PLACES.items()}
    return {"schedule": names[out[0].value], "ring": out[1].value, "xcd": out[2].value, "lpt": out[3].value,
            "place": places[out[4].value], "bn": out[5].value, "hpw": out[6].value}


def attn_device_clock(device: int = 0) -> tuple[int, int]:
    """C attn_device_clock: (compute units, peak shader clock in kHz) of a HIP device."""
    cu, khz = ctypes.c_int(0), ctypes.c_int(0)
    st = load().attn_device_clock(int(device), ctypes.byref(cu), ctypes.byref(khz))
    if st != ATTN_OK:
        raise AttnError(st)
    return cu.value, khz.value


def attn_mfma_ceiling(iters: int = 200000, stream=None) -> float:
    """C attn_mfma_ceiling: the sustained dense fp16 MFMA rate of the current device on random operands
    (TFLOP/s), a measurement aid.  `stream` as for attn_fwd_stream; the call waits for its timed launch."""
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else (stream or 0)
    out = ctypes.c_double(0.0)
    st = load().attn_mfma_ceiling(int(iters), handle, ctypes.byref(out))
    if st != ATTN_OK:
        raise AttnError(st)
    return out.value


def attn_mfma_ceiling_shape(shape: int, iters: int = 200000, stream=None) -> float:
    """C attn_mfma_ceiling_shape: attn_mfma_ceiling for `shape` 32 (32x32x16) or 16 (16x16x32)."""
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else (stream or 0)
    out = ctypes.c_double(0.0)
    st = load().attn_mfma_ceiling_shape(int(shape), int(iters), handle, ctypes.byref(out))
    if st != ATTN_OK:
        raise AttnError(st)
    return out.value


def gemm_f16_waves(a, b, c, M: int, N: int, K: int, b_layout: int, waves: int, stream) -> int:
    """C gemm_f16_waves: gemm_f16 with an explicit workgroup shape (waves 4 or 8; 0 the default)."""
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else (stream or 0)
    return load().gemm_f16_waves(_ptr(a), _ptr(b), _ptr(c), int(M), int(N), int(K), int(b_layout), int(waves),
                                 handle)


def gemm_f16(a, b, c, M: int, N: int, K: int, b_layout: int, stream) -> int:
    """C gemm_f16: C[M,N] = A[M,K] B (b_layout 0, B [K,N]) or A B^T (b_layout 1, B [N,K]).  `stream` as for
    attn_fwd_stream."""
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else (stream or 0)
    return load().gemm_f16(_ptr(a), _ptr(b), _ptr(c), int(M), int(N), int(K), int(b_layout), handle)


def attn_fwd_decode(q, k, v, o, lse, B: int, Sq: int, Sk: int, Hq: int, Hkv: int, D: int, causal: int,
                    scale: float, workspace, workspace_bytes: int, stream) -> int:
    """C attn_fwd_decode (split-KV path).  `workspace` is a tensor or raw device address of at least
    attn_decode_workspace_size(...) bytes; `stream` as for attn_fwd_stream."""
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else (stream or 0)
    return load().attn_fwd_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Sq, Sk, Hq, Hkv, D, int(causal),
                                  float(scale), _ptr(workspace), int(workspace_bytes), handle)


def attn_fwd_decode_split(q, k, v, o, lse, B: int, Sq: int, Sk: int, Hq: int, Hkv: int, D: int, causal: int,
                          scale: float, split_tiles: int, workspace, workspace_bytes: int, stream) -> int:
    """C attn_fwd_decode_split: attn_fwd_decode with an explicit split length (64-key tiles per split)."""
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else (stream or 0)
    return load().attn_fwd_decode_split(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Sq, Sk, Hq, Hkv, D,
                                        int(causal), float(scale), int(split_tiles), _ptr(workspace),
                                        int(workspace_bytes), handle)


def attn_decode_workspace_size(B: int, Sq: int, Sk: int, Hq: int, Hkv: int, D: int) -> int:
    return int(load().attn_decode_workspace_size(B, Sq, Sk, Hq, Hkv, D))


def attn_decode_workspace_size_split(B: int, Sq: int, Sk: int, Hq: int, Hkv: int, D: int, split_tiles: int) -> int:
    return int(load().attn_decode_workspace_size_split(B, Sq, Sk, Hq, Hkv, D, int(split_tiles)))


def variant_fields(variant) -> tuple:
    """(schedule, ring, xcd, lpt, place, bn, hpw) for attn_fwd_variant from None (all tuned), a schedule name,
    or a dict with any of the keys schedule (name or number), ring, xcd, lpt, place (name or number), bn
    (keys per K/V tile), hpw (heads per workgroup, wide schedule); missing fields are -1 (tuned)."""
    if variant is None:
        return (-1, -1, -1, -1, -1, -1, -1)
    if isinstance(variant, str):
        variant = {"schedule": variant}
    sched = variant.get("schedule", -1)
    if isinstance(sched, str):
        sched = SCHEDULES[sched]
    place = variant.get("place", -1)
    if isinstance(place, str):
        place = PLACES[place]
    return (int(sched), int(variant.get("ring", -1)), int(variant.get("xcd", -1)), int(variant.get("lpt", -1)),
            int(place), int(variant.get("bn", -1)), int(variant.get("hpw", -1)))


def attn_status_string(status: int) -> str:
    return load().attn_status_string(int(status)).decode()


def attn_version() -> int:
    return load().attn_version()


def forward(q, k, v, causal: bool = True, scale: float | None = None, out=None, lse=None, want_lse: bool = True,
            stream=None, variant=None):
    """Run the kernel on torch tensors q [B,Sq,Hq,D], k/v [B,Sk,Hkv,D] (fp16, contiguous, same GPU).

    Sk may differ from Sq (causal then aligns the last query row with the last key; see attn_fwd_ex).
    Returns (o, lse) with o [B,Sq,Hq,D] fp16 and lse [B,Hq,Sq] fp32 (None if not wanted).  Enqueues on
    `stream` (default: torch's current stream) and does not synchronise.  `variant` (see variant_fields)
    names a kernel variant through attn_fwd_variant; None runs the tuned one.
    """
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("%s must be a contiguous float16 tensor on a GPU" % name)
        if t.dim() != 4:
            raise ValueError("%s must be [B, S, H, D]" % name)
    B, S, Hq, D = q.shape
    Sk = k.shape[1]
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != D:
        raise ValueError("shape mismatch: q %s k %s v %s" % (tuple(q.shape), tuple(k.shape), tuple(v.shape)))
    if q.device != k.device or q.device != v.device:
        raise ValueError("q, k, v must be on the same device")
    Hkv = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if want_lse and lse is None:
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (B, Hq, S)):
        raise ValueError("lse must be a contiguous float32 [B, Hq, S] tensor")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    with torch.cuda.device(q.device):
        if variant is not None:
            st = attn_fwd_variant(q, k, v, out, lse, B, S, Sk, Hq, Hkv, D, int(bool(causal)), float(scale),
                                  *variant_fields(variant), stream)
        elif Sk == S:
            st = attn_fwd_stream(q, k, v, out, lse, B, S, Hq, Hkv, D, int(bool(causal)), float(scale), stream)
        else:
            st = attn_fwd_ex(q, k, v, out, lse, B, S, Sk, Hq, Hkv, D, int(bool(causal)), float(scale), stream)
    if st != ATTN_OK:
        raise AttnError(st)
    return out, lse


def matmul(a, b, b_layout: int = GEMM_B_KN, out=None, stream=None, waves: int = 0):
    """C = A B (b_layout 0, b [K, N]) or A B^T (b_layout 1, b [N, K]) on fp16 torch tensors, fp32 accumulation.

    a is [M, K]; all tensors contiguous float16 on one GPU.  Returns c [M, N] fp16.  Enqueues on `stream`
    (default: torch's current stream) and does not synchronise.  `waves` 4 or 8 picks the workgroup shape
    through gemm_f16_waves (0: the default).
    """
    import torch

    for name, t in (("a", a), ("b", b)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("%s must be a contiguous float16 tensor on a GPU" % name)
        if t.dim() != 2:
            raise ValueError("%s must be 2-D" % name)
    if b_layout not in (GEMM_B_KN, GEMM_B_NK):
        raise ValueError("b_layout must be 0 ([K, N]) or 1 ([N, K])")
    M, K = a.shape
    Kb, N = b.shape if b_layout == GEMM_B_KN else (b.shape[1], b.shape[0])
    if Kb != K:
        raise ValueError("shapes do not chain: a %s, b %s (b_layout %d)" % (tuple(a.shape), tuple(b.shape), b_layout))
    if a.device != b.device:
        raise ValueError("a and b must be on the same device")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=a.device)
    if out.dtype != torch.float16 or not out.is_contiguous() or tuple(out.shape) != (M, N):
        raise ValueError("out must be a contiguous float16 [M, N] tensor")
    if stream is None:
        stream = torch.cuda.current_stream(a.device)
    with torch.cuda.device(a.device):
        if waves:
            st = gemm_f16_waves(a, b, out, M, N, K, b_layout, waves, stream)
        else:
            st = gemm_f16(a, b, out, M, N, K, b_layout, stream)
    if st != ATTN_OK:
        raise AttnError(st)
    return out


def decode(q, k, v, causal: bool = True, scale: float | None = None, out=None, lse=None, want_lse: bool = True,
           workspace=None, stream=None, split_tiles: int = 0):
    """The split-KV path on torch tensors (same layout and result as forward()); allocates the workspace
    with torch unless one is given (then on `stream`, so torch's allocator does not hand the memory to other
    work before the kernels are done).  `split_tiles` > 0 fixes the split length (attn_fwd_decode_split).
    Returns (o, lse)."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("%s must be a contiguous float16 tensor on a GPU" % name)
        if t.dim() != 4:
            raise ValueError("%s must be [B, S, H, D]" % name)
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != D:
        raise ValueError("shape mismatch: q %s k %s v %s" % (tuple(q.shape), tuple(k.shape), tuple(v.shape)))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    torch_stream = stream if isinstance(stream, torch.cuda.Stream) else None
    if out is None:
        out = torch.empty_like(q)
    if want_lse and lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    need = attn_decode_workspace_size_split(B, Sq, Sk, Hq, Hkv, D, split_tiles)
    own_ws = workspace is None
    if own_ws:
        workspace = torch.empty((max(need, 16) + 15) // 16 * 4, dtype=torch.float32, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size() if hasattr(workspace, "numel") else need
    with torch.cuda.device(q.device):
        st = attn_fwd_decode_split(q, k, v, out, lse, B, Sq, Sk, Hq, Hkv, D, int(bool(causal)), float(scale),
                                   split_tiles, workspace, ws_bytes, stream)
    if st != ATTN_OK:
        raise AttnError(st)
    if own_ws and torch_stream is not None and torch_stream != torch.cuda.current_stream(q.device):
        # the workspace was allocated on the current stream but is used on another one
        workspace.record_stream(torch_stream)
    return out, lse
