"""Planted mistakes in the oracle must fail at least one pin (CPU only).

Each mutant is a one-line edit of a copy of oracle/attn_oracle.c, compiled to a
temporary library; the original source is never modified.
"""
import os

import pytest

from oracle import oracle as oracle_mod
from tests import oracle_pins as P

MUTANTS = {
    "gqa_map_modulo": ("const int c = h / g;", "const int c = h % Hkv;"),
    "causal_excludes_diagonal": ("J->causal ? i + 1 + off : Sk", "J->causal ? (i + off > 0 ? i + off : 1) : Sk"),
    "causal_one_key_too_many": ("J->causal ? i + 1 + off : Sk", "J->causal ? (i + 2 + off < Sk ? i + 2 + off : Sk) : Sk"),
    "causal_offset_dropped": ("J->causal ? i + 1 + off : Sk", "J->causal ? i + 1 : Sk"),
    "causal_offset_sign": ("const int off = J->Sk - J->Sq;", "const int off = J->Sq - J->Sk;"),
    "scale_dropped": ("scores[j] = J->sigma * dot;", "scores[j] = dot;"),
    "lse_without_max": ("J->lse[item] = m + log(l);", "J->lse[item] = log(l);"),
    "k_and_v_swapped": ("const double* kr = J->kd +", "const double* kr = J->vd +"),
    "no_normaliser": ("out[d] = acc[d] / l;", "out[d] = acc[d];"),
    "wrong_sign_in_exp": ("exp(scores[j] - m)", "exp(m - scores[j])"),
    "q_index_transposed": ("J->q[((int64_t)i * Hq + h) * D + d]", "J->q[((int64_t)h * J->Sq + i) * D + d]"),
    "dropped_first_d_term": ("for (int d = 0; d < D; ++d) dot +=", "for (int d = 1; d < D; ++d) dot +="),
    "v_row_off_by_one": ("const double* vr = J->vd + ((int64_t)j * Hkv + c) * D;",
                         "const double* vr = J->vd + ((int64_t)(j + 1 < Sk ? j + 1 : j) * Hkv + c) * D;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle_mod.SRC).read()
    assert src.count(old) == 1, "mutation anchor not found exactly once: %r" % old
    msrc = tmp_path / ("mutant_%s.c" % name)
    msrc.write_text(src.replace(old, new))
    lib = oracle_mod.build(str(msrc), str(tmp_path / ("mutant_%s.so" % name)))
    orc = oracle_mod.Oracle(lib)
    failed = []
    for pin in P.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, RuntimeError, FloatingPointError, ValueError):
            failed.append(pin.__name__)
    assert failed, "no pin caught mutant %s" % name
    print("%s caught by %s" % (name, ", ".join(failed)))


def test_unmutated_copy_passes_every_pin(tmp_path):
    src = open(oracle_mod.SRC).read()
    csrc = tmp_path / "copy.c"
    csrc.write_text(src)
    orc = oracle_mod.Oracle(oracle_mod.build(str(csrc), str(tmp_path / "copy.so")))
    for pin in P.ALL_PINS:
        pin(orc)
    assert os.path.exists(oracle_mod.SRC)
