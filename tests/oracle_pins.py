"""Pins for the fp64 attention oracle: checks against things other than itself.

Each pin takes an `Oracle` and raises AssertionError when the oracle disagrees
with a closed form, an invariant, a library routine, a hand-worked example or
brute force.  They are written so that a plausible mistake anywhere in the
oracle (wrong GQA head map, causal off-by-one, dropped scale, missing max in
the LSE, swapped K/V roles, wrong normaliser) fails at least one of them;
tests/test_oracle_mutants.py plants such mistakes and checks exactly that.
"""
from __future__ import annotations

import json
import math
import os
import struct

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "handworked.json")


def f32(x: float) -> float:
    return struct.unpack("<f", struct.pack("<f", x))[0]


def f32_bits(s: str) -> float:
    return struct.unpack("<f", struct.pack("<I", int(s, 16)))[0]


def rand_qkv(rng, B, S, Hq, Hkv, D, std=1.0):
    q = (rng.standard_normal((B, S, Hq, D)) * std).astype(np.float16)
    k = (rng.standard_normal((B, S, Hkv, D)) * std).astype(np.float16)
    v = rng.standard_normal((B, S, Hkv, D)).astype(np.float16)
    return q, k, v


# ---------------------------------------------------------------- golden

def pin_handworked(orc):
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q = np.array(c["q"], dtype=np.float16)
        k = np.array(c["k"], dtype=np.float16)
        v = np.array(c["v"], dtype=np.float16)
        assert q.shape == (c["S"], c["Hq"], c["D"])
        scale = f32_bits(c["scale_bits"])
        O, L = orc.full(q[None], k[None], v[None], bool(c["causal"]), scale)
        np.testing.assert_allclose(O[0], np.array(c["expected_o"]), rtol=1e-7, atol=1e-7, err_msg=c["name"])
        np.testing.assert_allclose(L[0], np.array(c["expected_lse"]), rtol=1e-7, atol=1e-7, err_msg=c["name"])


# ---------------------------------------------------------------- library routine

def torch_reference(q, k, v, causal, scale):
    """float64 torch: scaled_dot_product_attention with K/V heads repeated g times, and
    logsumexp of the masked scaled scores.  Returns (O [B,S,Hq,D], LSE [B,Hq,S])."""
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    g = Hq // Hkv
    qt = torch.from_numpy(q.astype(np.float64)).permute(0, 2, 1, 3)  # [B,Hq,S,D]
    kt = torch.from_numpy(k.astype(np.float64)).permute(0, 2, 1, 3).repeat_interleave(g, dim=1)
    vt = torch.from_numpy(v.astype(np.float64)).permute(0, 2, 1, 3).repeat_interleave(g, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=bool(causal), scale=float(scale))
    s = torch.matmul(qt, kt.transpose(-1, -2).contiguous()) * float(scale)
    if causal:
        mask = torch.ones(S, S, dtype=torch.bool).tril()
        s = s.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return o.permute(0, 2, 1, 3).numpy(), lse.numpy()


SDPA_SHAPES = [
    # B, S, Hq, Hkv, D
    (1, 1, 1, 1, 1),
    (2, 2, 2, 1, 3),
    (1, 3, 4, 2, 8),
    (2, 17, 8, 2, 16),
    (1, 64, 4, 1, 128),
    (1, 129, 8, 8, 64),
    (2, 33, 8, 1, 128),
    (1, 40, 4, 2, 256),
]


def pin_torch_sdpa(orc, seed=11):
    rng = np.random.default_rng(seed)
    for B, S, Hq, Hkv, D in SDPA_SHAPES:
        for causal in (True, False):
            q, k, v = rand_qkv(rng, B, S, Hq, Hkv, D)
            scale = f32(float(rng.uniform(0.05, 0.6)))
            O, L = orc.full(q, k, v, causal, scale)
            Ot, Lt = torch_reference(q, k, v, causal, scale)
            tag = "B%d S%d Hq%d Hkv%d D%d causal%d" % (B, S, Hq, Hkv, D, causal)
            np.testing.assert_allclose(O, Ot, rtol=1e-10, atol=1e-11, err_msg=tag)
            np.testing.assert_allclose(L, Lt, rtol=1e-10, atol=1e-11, err_msg=tag)


# ---------------------------------------------------------------- closed forms

def pin_constant_v(orc, seed=12):
    """Every V row of a KV head equals the same vector u: O = u for any Q, K."""
    rng = np.random.default_rng(seed)
    B, S, Hq, Hkv, D = 2, 23, 4, 2, 16
    q, k, _ = rand_qkv(rng, B, S, Hq, Hkv, D)
    u = rng.standard_normal((B, 1, Hkv, D)).astype(np.float16)
    v = np.broadcast_to(u, (B, S, Hkv, D)).copy()
    g = Hq // Hkv
    for causal in (True, False):
        O, _ = orc.full(q, k, v, causal, 0.37)
        want = np.repeat(u.astype(np.float64), g, axis=2)  # head h -> kv head h // g
        np.testing.assert_allclose(O, np.broadcast_to(want, O.shape), rtol=0, atol=1e-14)


def pin_zero_q(orc, seed=13):
    """Q = 0: uniform weights over the allowed keys. O_i = mean of V over A(i); LSE_i = ln |A(i)|."""
    rng = np.random.default_rng(seed)
    B, S, Hq, Hkv, D = 1, 19, 4, 2, 8
    _, k, v = rand_qkv(rng, B, S, Hq, Hkv, D)
    q = np.zeros((B, S, Hq, D), dtype=np.float16)
    g = Hq // Hkv
    vd = v.astype(np.float64)
    for causal in (True, False):
        O, L = orc.full(q, k, v, causal, 0.5)
        for i in range(S):
            n = i + 1 if causal else S
            mean = vd[0, :n].mean(axis=0)  # [Hkv, D]
            for h in range(Hq):
                np.testing.assert_allclose(O[0, i, h], mean[h // g], rtol=0, atol=1e-14)
                assert abs(L[0, h, i] - math.log(n)) < 1e-14


def pin_first_causal_row(orc, seed=14):
    """Causal row 0 sees only key 0: O = V[0], LSE = scale * q0.k0."""
    rng = np.random.default_rng(seed)
    B, S, Hq, Hkv, D = 2, 9, 8, 2, 32
    q, k, v = rand_qkv(rng, B, S, Hq, Hkv, D)
    scale = f32(0.125)
    O, L = orc.full(q, k, v, True, scale)
    g = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            c = h // g
            assert np.array_equal(O[b, 0, h], v[b, 0, c].astype(np.float64))
            dot = math.fsum(float(x) * float(y) for x, y in zip(q[b, 0, h].astype(np.float64),
                                                                 k[b, 0, c].astype(np.float64)))
            assert abs(L[b, h, 0] - scale * dot) < 1e-12


def pin_gqa_constant_heads(orc, seed=15):
    """V of KV head c filled with c+1: output head h equals floor(h / g) + 1 (consecutive heads share)."""
    rng = np.random.default_rng(seed)
    for Hq, Hkv in ((8, 2), (8, 4), (6, 3), (4, 1)):
        B, S, D = 1, 11, 4
        q, k, _ = rand_qkv(rng, B, S, Hq, Hkv, D)
        v = np.empty((B, S, Hkv, D), dtype=np.float16)
        for c in range(Hkv):
            v[:, :, c, :] = c + 1
        g = Hq // Hkv
        for causal in (True, False):
            O, _ = orc.full(q, k, v, causal, 0.3)
            for h in range(Hq):
                np.testing.assert_allclose(O[0, :, h, :], h // g + 1, rtol=0, atol=1e-13)


def pin_large_scale_argmax(orc, seed=16):
    """scale = 1e4 with well-separated scores: softmax is one-hot on the argmax key."""
    rng = np.random.default_rng(seed)
    B, S, Hq, Hkv, D = 1, 12, 2, 1, 4
    q, k, v = rand_qkv(rng, B, S, Hq, Hkv, D)
    scale = f32(1e4)
    for causal in (True, False):
        O, L = orc.full(q, k, v, causal, scale)
        for h in range(Hq):
            for i in range(S):
                n = i + 1 if causal else S
                s = np.array([float(np.dot(q[0, i, h].astype(np.float64), k[0, j, 0].astype(np.float64)))
                              for j in range(n)])
                order = np.sort(s)
                if n > 1 and order[-1] - order[-2] < 5e-3:
                    continue  # not separated enough for a one-hot limit
                j = int(np.argmax(s))
                np.testing.assert_allclose(O[0, i, h], v[0, j, 0].astype(np.float64), rtol=0, atol=1e-12)
                assert abs(L[0, h, i] - scale * s[j]) <= 1e-9 * max(1.0, abs(scale * s[j]))


# ---------------------------------------------------------------- invariants

def pin_causal_is_prefix(orc, seed=17):
    """Causal row i equals non-causal attention over the prefix keys 0..i."""
    rng = np.random.default_rng(seed)
    B, S, Hq, Hkv, D = 1, 14, 4, 2, 8
    q, k, v = rand_qkv(rng, B, S, Hq, Hkv, D)
    Oc, Lc = orc.full(q, k, v, True, 0.4)
    for i in (0, 1, 5, 13):
        On, Ln = orc.full(q[:, :i + 1], k[:, :i + 1], v[:, :i + 1], False, 0.4)
        np.testing.assert_allclose(Oc[:, i], On[:, i], rtol=0, atol=1e-14)
        np.testing.assert_allclose(Lc[:, :, i], Ln[:, :, i], rtol=0, atol=1e-14)


def pin_key_shift(orc, seed=18):
    """Adding the same vector u to every key leaves O unchanged and shifts LSE_i by scale * q_i.u.
    Inputs sit on a coarse grid so K + u stays exactly representable in fp16."""
    rng = np.random.default_rng(seed)
    B, S, Hq, Hkv, D = 1, 10, 4, 2, 8
    q = (rng.integers(-8, 9, (B, S, Hq, D)) / 8).astype(np.float16)
    k = (rng.integers(-8, 9, (B, S, Hkv, D)) / 8).astype(np.float16)
    v = rng.standard_normal((B, S, Hkv, D)).astype(np.float16)
    u = (rng.integers(-4, 5, (Hkv, D)) / 4).astype(np.float16)
    k2 = (k.astype(np.float64) + u.astype(np.float64)[None, None]).astype(np.float16)
    assert np.array_equal(k2.astype(np.float64), k.astype(np.float64) + u.astype(np.float64)[None, None])
    scale = 0.25
    g = Hq // Hkv
    for causal in (True, False):
        O1, L1 = orc.full(q, k, v, causal, scale)
        O2, L2 = orc.full(q, k2, v, causal, scale)
        np.testing.assert_allclose(O2, O1, rtol=0, atol=1e-12)
        for h in range(Hq):
            shift = scale * (q[0, :, h].astype(np.float64) @ u[h // g].astype(np.float64))
            np.testing.assert_allclose(L2[0, h] - L1[0, h], shift, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- brute force

def brute_force(q, k, v, causal, scale):
    """Pure Python, without the max shift: w_j = exp(s_j) directly, sums by math.fsum.
    Only for tiny inputs with small scores (no overflow)."""
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    g = Hq // Hkv
    O = np.zeros((B, S, Hq, D))
    L = np.zeros((B, Hq, S))
    qd, kd, vd = q.astype(np.float64), k.astype(np.float64), v.astype(np.float64)
    for b in range(B):
        for h in range(Hq):
            c = h // g
            for i in range(S):
                keys = range(i + 1) if causal else range(S)
                w = [math.exp(scale * math.fsum(qd[b, i, h, d] * kd[b, j, c, d] for d in range(D))) for j in keys]
                tot = math.fsum(w)
                for d in range(D):
                    O[b, i, h, d] = math.fsum(wj * vd[b, j, c, d] for wj, j in zip(w, keys)) / tot
                L[b, h, i] = math.log(tot)
    return O, L


def pin_brute_force(orc, seed=19):
    rng = np.random.default_rng(seed)
    for B, S, Hq, Hkv, D in ((1, 1, 1, 1, 1), (2, 3, 2, 1, 3), (1, 5, 4, 2, 8), (1, 17, 2, 2, 4), (1, 6, 8, 4, 128)):
        q, k, v = rand_qkv(rng, B, S, Hq, Hkv, D)
        for causal in (True, False):
            scale = f32(float(rng.uniform(0.05, 0.5)))
            O, L = orc.full(q, k, v, causal, scale)
            Ob, Lb = brute_force(q, k, v, causal, scale)
            np.testing.assert_allclose(O, Ob, rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(L, Lb, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- Sq != Sk (bottom-right causal alignment)

def rand_qkv_rect(rng, B, Sq, Sk, Hq, Hkv, D):
    q = rng.standard_normal((B, Sq, Hq, D)).astype(np.float16)
    k = rng.standard_normal((B, Sk, Hkv, D)).astype(np.float16)
    v = rng.standard_normal((B, Sk, Hkv, D)).astype(np.float16)
    return q, k, v


def torch_reference_rect(q, k, v, causal, scale):
    """float64 torch for Sq != Sk: scaled_dot_product_attention with an explicit boolean mask (query i
    may attend key j iff j <= i + Sk - Sq when causal), and logsumexp of the masked scaled scores."""
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    g = Hq // Hkv
    qt = torch.from_numpy(q.astype(np.float64)).permute(0, 2, 1, 3)
    kt = torch.from_numpy(k.astype(np.float64)).permute(0, 2, 1, 3).repeat_interleave(g, dim=1)
    vt = torch.from_numpy(v.astype(np.float64)).permute(0, 2, 1, 3).repeat_interleave(g, dim=1)
    allowed = torch.ones(Sq, Sk, dtype=torch.bool)
    if causal:
        allowed = torch.arange(Sk)[None, :] <= torch.arange(Sq)[:, None] + (Sk - Sq)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=allowed, scale=float(scale))
    s = torch.matmul(qt, kt.transpose(-1, -2).contiguous()) * float(scale)
    lse = torch.logsumexp(s.masked_fill(~allowed, float("-inf")), dim=-1)
    return o.permute(0, 2, 1, 3).numpy(), lse.numpy()


RECT_SHAPES = [
    # B, Sq, Sk, Hq, Hkv, D
    (1, 1, 7, 2, 1, 8),
    (2, 3, 17, 4, 2, 16),
    (1, 16, 64, 8, 2, 128),
    (1, 33, 100, 4, 4, 64),
]


def pin_torch_sdpa_rect(orc, seed=21):
    rng = np.random.default_rng(seed)
    for B, Sq, Sk, Hq, Hkv, D in RECT_SHAPES:
        for causal in (True, False):
            q, k, v = rand_qkv_rect(rng, B, Sq, Sk, Hq, Hkv, D)
            scale = f32(float(rng.uniform(0.05, 0.6)))
            O, L = orc.full(q, k, v, causal, scale)
            Ot, Lt = torch_reference_rect(q, k, v, causal, scale)
            tag = "B%d Sq%d Sk%d Hq%d Hkv%d D%d causal%d" % (B, Sq, Sk, Hq, Hkv, D, causal)
            np.testing.assert_allclose(O, Ot, rtol=1e-10, atol=1e-11, err_msg=tag)
            np.testing.assert_allclose(L, Lt, rtol=1e-10, atol=1e-11, err_msg=tag)
    # more query rows than keys, non-causal
    q, k, v = rand_qkv_rect(rng, 1, 9, 4, 2, 1, 8)
    O, L = orc.full(q, k, v, False, f32(0.3))
    Ot, Lt = torch_reference_rect(q, k, v, False, f32(0.3))
    np.testing.assert_allclose(O, Ot, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(L, Lt, rtol=1e-10, atol=1e-11)


def pin_zero_q_rect(orc, seed=22):
    """Q = 0 with Sq < Sk, causal: query row i averages V over keys 0..i+Sk-Sq; LSE = ln(i+1+Sk-Sq)."""
    rng = np.random.default_rng(seed)
    B, Sq, Sk, Hq, Hkv, D = 1, 6, 15, 4, 2, 8
    _, k, v = rand_qkv_rect(rng, B, Sq, Sk, Hq, Hkv, D)
    q = np.zeros((B, Sq, Hq, D), dtype=np.float16)
    O, L = orc.full(q, k, v, True, 0.5)
    vd = v.astype(np.float64)
    g = Hq // Hkv
    for i in range(Sq):
        n = i + 1 + Sk - Sq
        mean = vd[0, :n].mean(axis=0)
        for h in range(Hq):
            np.testing.assert_allclose(O[0, i, h], mean[h // g], rtol=0, atol=1e-14)
            assert abs(L[0, h, i] - math.log(n)) < 1e-14


def pin_suffix_of_square(orc, seed=23):
    """Causal with Sq < Sk equals the last Sq rows of the square Sk x Sk problem whose last Sq query
    rows are the given ones (the square case is pinned on its own above)."""
    rng = np.random.default_rng(seed)
    B, Sq, Sk, Hq, Hkv, D = 2, 5, 21, 4, 2, 16
    q, k, v = rand_qkv_rect(rng, B, Sq, Sk, Hq, Hkv, D)
    qfull = np.concatenate([rng.standard_normal((B, Sk - Sq, Hq, D)).astype(np.float16), q], axis=1)
    O, L = orc.full(q, k, v, True, 0.35)
    Of, Lf = orc.full(qfull, k, v, True, 0.35)
    np.testing.assert_allclose(O, Of[:, Sk - Sq:], rtol=0, atol=1e-14)
    np.testing.assert_allclose(L, Lf[:, :, Sk - Sq:], rtol=0, atol=1e-14)


def brute_force_rect(q, k, v, causal, scale):
    """brute_force for Sq != Sk (bottom-right causal alignment)."""
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    g = Hq // Hkv
    O = np.zeros((B, Sq, Hq, D))
    L = np.zeros((B, Hq, Sq))
    qd, kd, vd = q.astype(np.float64), k.astype(np.float64), v.astype(np.float64)
    for b in range(B):
        for h in range(Hq):
            c = h // g
            for i in range(Sq):
                keys = range(i + 1 + Sk - Sq) if causal else range(Sk)
                w = [math.exp(scale * math.fsum(qd[b, i, h, d] * kd[b, j, c, d] for d in range(D))) for j in keys]
                tot = math.fsum(w)
                for d in range(D):
                    O[b, i, h, d] = math.fsum(wj * vd[b, j, c, d] for wj, j in zip(w, keys)) / tot
                L[b, h, i] = math.log(tot)
    return O, L


def pin_brute_force_rect(orc, seed=24):
    rng = np.random.default_rng(seed)
    for B, Sq, Sk, Hq, Hkv, D in ((1, 1, 3, 1, 1, 2), (1, 4, 9, 2, 1, 8), (2, 3, 5, 4, 2, 4)):
        q, k, v = rand_qkv_rect(rng, B, Sq, Sk, Hq, Hkv, D)
        for causal in (True, False):
            scale = f32(float(rng.uniform(0.05, 0.5)))
            O, L = orc.full(q, k, v, causal, scale)
            Ob, Lb = brute_force_rect(q, k, v, causal, scale)
            np.testing.assert_allclose(O, Ob, rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(L, Lb, rtol=1e-12, atol=1e-13)


ALL_PINS = [pin_handworked, pin_torch_sdpa, pin_constant_v, pin_zero_q, pin_first_causal_row, pin_gqa_constant_heads,
            pin_large_scale_argmax, pin_causal_is_prefix, pin_key_shift, pin_brute_force, pin_torch_sdpa_rect,
            pin_zero_q_rect, pin_suffix_of_square, pin_brute_force_rect]
