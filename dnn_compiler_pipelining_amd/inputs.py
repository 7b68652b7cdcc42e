"""Seeded synthetic inputs for the attention forward pass and the fp16 GEMM.

This module holds no attention or GEMM arithmetic.  It is the only code shared
by the GPU path's tests/bench and the oracle's callers: both sides read the
exact fp16 values produced here.

Workloads: the FlashAttention evaluation of PipeThreader runs LLaMA3-8B and
LLaMA3-70B head shapes at sequence lengths 512..8k and batch sizes 1 and 64
(page "PipeThreader ... (OSDI 2025)" summary, section "实验与结果", citing the
paper's section 6.2 / Fig.12).  No dataset is involved; the heads enter only as
shapes: D = 128, Hq/Hkv = 32/8 (8B) or 64/8 (70B).

Recipe: for tensor t in {Q: 0, K: 1, V: 2} and batch entry b, a CPU
torch.Generator seeded with base * 1_000_003 + t * 65_537 + b draws
torch.randn((S, H_t, D), float32), which is rounded to fp16 (round to nearest
even).  Seeding per (tensor, batch entry) lets a checker regenerate any batch
slice on its own, and lets slices be generated in parallel.
"""
from __future__ import annotations

import struct
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import torch

Q, K, V = 0, 1, 2

# fp32 value of 1/sqrt(128), the softmax scale every workload uses.
SCALE_D128 = struct.unpack("<f", struct.pack("<I", 0x3DB504F3))[0]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    S: int
    Hq: int
    Hkv: int
    D: int
    causal: bool
    seed: int
    scale: float = SCALE_D128

    @property
    def flops(self) -> float:
        """Metric FLOPs: 2 * B * Hq * S^2 * D (QK^T and PV over the causal half)."""
        return 2.0 * self.B * self.Hq * self.S * self.S * self.D

    def heads(self, t: int) -> int:
        return self.Hq if t == Q else self.Hkv

    def describe(self) -> dict:
        return {"workload": self.name, "B": self.B, "S": self.S, "Hq": self.Hq, "Hkv": self.Hkv, "D": self.D,
                "causal": self.causal, "layout": "[B,S,H,D] fp16 in/out, LSE [B,Hq,S] fp32",
                "scale": self.scale, "seed": self.seed}


WORKLOADS = [
    Workload("llama3-8b_b1_s512", 1, 512, 32, 8, 128, True, 1),
    Workload("llama3-8b_b1_s8192", 1, 8192, 32, 8, 128, True, 2),
    Workload("llama3-70b_b1_s8192", 1, 8192, 64, 8, 128, True, 3),
    Workload("llama3-8b_b64_s2048", 64, 2048, 32, 8, 128, True, 4),
    Workload("llama3-70b_b64_s8192", 64, 8192, 64, 8, 128, True, 5),
]
BY_NAME = {w.name: w for w in WORKLOADS}


def slice_seed(base: int, tensor: int, b: int) -> int:
    return base * 1_000_003 + tensor * 65_537 + b


def make_slice(S: int, H: int, D: int, base: int, tensor: int, b: int) -> torch.Tensor:
    """One batch entry of one tensor: CPU fp16 [S, H, D], N(0,1) rounded to fp16."""
    g = torch.Generator(device="cpu").manual_seed(slice_seed(base, tensor, b))
    return torch.randn((S, H, D), generator=g, dtype=torch.float32).to(torch.float16)


def _threads() -> int:
    import os
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def make_tensor(B: int, S: int, H: int, D: int, base: int, tensor: int, device="cpu") -> torch.Tensor:
    """Full [B, S, H, D] fp16 tensor, batch slices generated in parallel and written into place."""
    out = torch.empty((B, S, H, D), dtype=torch.float16, device=device)

    def fill(b):
        x = make_slice(S, H, D, base, tensor, b)
        out[b].copy_(x, non_blocking=False)
        return b

    if B == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(B)))
    return out


def make_inputs(w: Workload, device="cpu"):
    """(q, k, v) for a workload on `device` ([B,S,Hq,D], [B,S,Hkv,D], [B,S,Hkv,D] fp16)."""
    q = make_tensor(w.B, w.S, w.Hq, w.D, w.seed, Q, device)
    k = make_tensor(w.B, w.S, w.Hkv, w.D, w.seed, K, device)
    v = make_tensor(w.B, w.S, w.Hkv, w.D, w.seed, V, device)
    return q, k, v


def make_batch_cpu(w: Workload, b: int):
    """(q, k, v) of batch entry b on the CPU: [S,Hq,D], [S,Hkv,D], [S,Hkv,D] fp16."""
    return (make_slice(w.S, w.Hq, w.D, w.seed, Q, b), make_slice(w.S, w.Hkv, w.D, w.seed, K, b),
            make_slice(w.S, w.Hkv, w.D, w.seed, V, b))


# ---------------------------------------------------------------- GEMM inputs
#
# The fp16 GEMM runs the "8k MatMul" workload that PipeThreader compiles and
# whose hardware-scheduled tensor-core utilisation it quotes (page "PipeThreader
# ... (OSDI 2025)" summary, sections "问题与动机" and "实验与结果", citing the
# paper's section 6.4 / Table 4): M = N = K = 8192.
#
# Recipe: matrix t in {A: 0, B: 1} is drawn by a CPU torch.Generator seeded
# with base * 1_000_003 + t * 65_537 + 7_919.  dist "normal": torch.randn
# float32 rounded to fp16.  dist "int": integers uniform in [-lim, lim]
# (torch.randint), stored as fp16; with these every partial sum of a dot
# product of length K <= 2^24 / lim^2 is an integer below 2^24, so fp32
# accumulation is exact in any order.

MAT_A, MAT_B = 0, 1
B_KN, B_NK = 0, 1  # B stored [K, N] (C = A B) or [N, K] (C = A B^T, the linear-layer weight layout)


@dataclass(frozen=True)
class GemmWorkload:
    name: str
    M: int
    N: int
    K: int
    b_layout: int
    seed: int
    dist: str = "normal"
    lim: int = 0

    @property
    def flops(self) -> float:
        """2 * M * N * K."""
        return 2.0 * self.M * self.N * self.K

    def b_shape(self):
        return (self.K, self.N) if self.b_layout == B_KN else (self.N, self.K)

    def describe(self) -> dict:
        return {"workload": self.name, "M": self.M, "N": self.N, "K": self.K,
                "b_layout": "B[K,N], C = A B" if self.b_layout == B_KN else "B[N,K], C = A B^T",
                "layout": "row-major fp16 A[M,K], fp16 C[M,N], fp32 accumulation",
                "dist": self.dist if self.dist == "normal" else "int[-%d,%d]" % (self.lim, self.lim),
                "seed": self.seed}


GEMM_WORKLOADS = [
    GemmWorkload("gemm_8k_nn", 8192, 8192, 8192, B_KN, 11),
    GemmWorkload("gemm_8k_nt", 8192, 8192, 8192, B_NK, 12),
]
GEMM_BY_NAME = {w.name: w for w in GEMM_WORKLOADS}


def make_matrix(rows: int, cols: int, base: int, which: int, dist: str = "normal", lim: int = 0,
                device="cpu") -> torch.Tensor:
    """CPU-generated fp16 [rows, cols] matrix (see the recipe above), moved to `device`."""
    g = torch.Generator(device="cpu").manual_seed(base * 1_000_003 + which * 65_537 + 7_919)
    if dist == "normal":
        x = torch.randn((rows, cols), generator=g, dtype=torch.float32).to(torch.float16)
    elif dist == "int":
        if lim < 1:
            raise ValueError("dist 'int' needs lim >= 1")
        x = torch.randint(-lim, lim + 1, (rows, cols), generator=g, dtype=torch.int32).to(torch.float16)
    else:
        raise ValueError("dist must be 'normal' or 'int'")
    return x if device == "cpu" else x.to(device)


def make_gemm_inputs(w: GemmWorkload, device="cpu"):
    """(a, b) for a GEMM workload: a [M, K], b [K, N] or [N, K] by w.b_layout, fp16."""
    a = make_matrix(w.M, w.K, w.seed, MAT_A, w.dist, w.lim, device)
    br, bc = w.b_shape()
    b = make_matrix(br, bc, w.seed, MAT_B, w.dist, w.lim, device)
    return a, b


# ---------------------------------------------------------------- decode inputs
#
# Single-token decode at LLaMA3-70B head shapes against an 8192-key cache (the
# pages' longest FlashAttention sequence), batch 64: the split-KV path
# (attn_fwd_decode).  Q, K and V follow the attention recipe above, with
# per-(tensor, batch entry) seeds; Q has Sq rows and K/V have Sk rows.


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    B: int
    Sq: int
    Sk: int
    Hq: int
    Hkv: int
    D: int
    causal: bool
    seed: int
    scale: float = SCALE_D128

    @property
    def bytes(self) -> float:
        """Algorithmic HBM bytes: K and V read once, Q read, O written (fp16), LSE written (fp32)."""
        return 2.0 * 2 * self.B * self.Sk * self.Hkv * self.D + 2.0 * 2 * self.B * self.Sq * self.Hq * self.D + \
            4.0 * self.B * self.Hq * self.Sq

    def describe(self) -> dict:
        return {"workload": self.name, "B": self.B, "Sq": self.Sq, "Sk": self.Sk, "Hq": self.Hq, "Hkv": self.Hkv,
                "D": self.D, "causal": self.causal, "path": "attn_fwd_decode (split-KV + combine)",
                "layout": "[B,S,H,D] fp16 in/out, LSE [B,Hq,Sq] fp32", "scale": self.scale, "seed": self.seed}


DECODE_WORKLOADS = [DecodeWorkload("llama3-70b_decode_b64_s8192", 64, 1, 8192, 64, 8, 128, True, 21)]
DECODE_BY_NAME = {w.name: w for w in DECODE_WORKLOADS}


def make_decode_inputs(w: DecodeWorkload, device="cpu"):
    """(q, k, v): [B,Sq,Hq,D], [B,Sk,Hkv,D], [B,Sk,Hkv,D] fp16."""
    return (make_tensor(w.B, w.Sq, w.Hq, w.D, w.seed, Q, device), make_tensor(w.B, w.Sk, w.Hkv, w.D, w.seed, K, device),
            make_tensor(w.B, w.Sk, w.Hkv, w.D, w.seed, V, device))


# ---------------------------------------------------------------- attention variants at the same boundary
#
# Shapes of the variants the same entry points serve beyond the causal square workloads: non-causal,
# sequence lengths off the tile sizes, chunked prefill (Sq < Sk, bottom-right causal mask) and head
# dimensions 64 and 256, at the workloads' head counts.  `bench.py --variants` times them; the GPU
# tests check sampled rows of each against the oracle.  Same recipe as above; the scale is the fp32
# value of 1/sqrt(D).

def scale_for(D: int) -> float:
    """fp32 value of 1/sqrt(D) for D in {64, 128, 256}."""
    return {64: 0.125, 128: SCALE_D128, 256: 0.0625}[D]


@dataclass(frozen=True)
class VariantShape:
    name: str
    B: int
    Sq: int
    Sk: int
    Hq: int
    Hkv: int
    D: int
    causal: bool
    seed: int

    @property
    def scale(self) -> float:
        return scale_for(self.D)

    @property
    def pairs(self) -> int:
        """(query, key) pairs a (batch, head) computes: Sq * Sk, or under the bottom-right causal mask the
        sum over rows i of min(Sk, i + Sk - Sq + 1)."""
        if not self.causal:
            return self.Sq * self.Sk
        off = self.Sk - self.Sq
        return sum(min(self.Sk, i + off + 1) for i in range(self.Sq))

    @property
    def flops(self) -> float:
        """4 * D FLOPs per computed (query, key) pair (QK^T and PV), over all batch entries and heads."""
        return 4.0 * self.D * self.B * self.Hq * self.pairs

    def describe(self) -> dict:
        return {"workload": self.name, "B": self.B, "Sq": self.Sq, "Sk": self.Sk, "Hq": self.Hq, "Hkv": self.Hkv,
                "D": self.D, "causal": self.causal, "layout": "[B,S,H,D] fp16 in/out, LSE [B,Hq,Sq] fp32",
                "scale": self.scale, "seed": self.seed}


VARIANT_SHAPES = [
    VariantShape("llama3-70b_b16_s8192_noncausal", 16, 8192, 8192, 64, 8, 128, False, 61),
    VariantShape("llama3-70b_b64_s8000", 64, 8000, 8000, 64, 8, 128, True, 62),
    VariantShape("llama3-8b_b64_s2000", 64, 2000, 2000, 32, 8, 128, True, 63),
    VariantShape("llama3-70b_b64_chunk2048_of_8192", 64, 2048, 8192, 64, 8, 128, True, 64),
    VariantShape("d64_b16_s8192", 16, 8192, 8192, 32, 8, 64, True, 65),
    VariantShape("d64_b16_s8192_noncausal", 16, 8192, 8192, 32, 8, 64, False, 66),
    VariantShape("d256_b16_s8192", 16, 8192, 8192, 32, 8, 256, True, 67),
    VariantShape("d256_b16_s8192_noncausal", 16, 8192, 8192, 32, 8, 256, False, 68),
]
VARIANT_BY_NAME = {w.name: w for w in VARIANT_SHAPES}


def make_variant_inputs(w: VariantShape, device="cpu"):
    """(q, k, v): [B,Sq,Hq,D], [B,Sk,Hkv,D], [B,Sk,Hkv,D] fp16."""
    return (make_tensor(w.B, w.Sq, w.Hq, w.D, w.seed, Q, device), make_tensor(w.B, w.Sk, w.Hkv, w.D, w.seed, K, device),
            make_tensor(w.B, w.Sk, w.Hkv, w.D, w.seed, V, device))


def make_variant_batch_cpu(w: VariantShape, b: int):
    """(q, k, v) of batch entry b on the CPU: [Sq,Hq,D], [Sk,Hkv,D], [Sk,Hkv,D] fp16."""
    return (make_slice(w.Sq, w.Hq, w.D, w.seed, Q, b), make_slice(w.Sk, w.Hkv, w.D, w.seed, K, b),
            make_slice(w.Sk, w.Hkv, w.D, w.seed, V, b))
