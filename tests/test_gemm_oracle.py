"""The fp64 GEMM oracle against its pins, and planted mistakes against the pins (CPU only)."""
import importlib.util

import pytest

from oracle import gemm_oracle
from tests import gemm_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(gemm_oracle)


# one-line edits of a copy of oracle/gemm_oracle.py; the original is never modified
MUTANTS = {
    "nk_layout_not_transposed": ("        return b64.T", "        return b64"),
    "kn_layout_transposed": ("    if b_layout == B_KN:\n        return b64\n", "    if b_layout == B_KN:\n        return b64.T\n"),
    "last_k_term_dropped": ("    return a64 @ b64\n", "    return a64[:, :-1] @ b64[:-1]\n"),
    "operands_swapped": ("    return a64 @ b64\n", "    return (b64.T @ a64.T)\n"),
    "double_rounding_through_fp32": ("np.asarray(c, dtype=np.float64).astype(np.float16)",
                                     "np.asarray(c, dtype=np.float32).astype(np.float16)"),
    "sampled_rows_shifted": ("[np.asarray(rows, dtype=np.int64)].astype(np.float64)",
                             "[(np.asarray(rows, dtype=np.int64) + 1) % np.asarray(a).shape[0]].astype(np.float64)"),
    "abs_products_signed_b": ("@ np.abs(_b_as_kn(b, b_layout))", "@ _b_as_kn(b, b_layout)"),
    "a_rounded_to_int": ("a64 = np.asarray(a, dtype=np.float16).astype(np.float64)\n    b64",
                         "a64 = np.rint(np.asarray(a, dtype=np.float16).astype(np.float64))\n    b64"),
}


def load_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(gemm_oracle.__file__).read()
    assert src.count(old) == 1, "mutation anchor not found exactly once: %r" % old
    path = tmp_path / ("gemm_mutant_%s.py" % name)
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("gemm_mutant_%s" % name, str(path))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    mod = load_mutant(name, tmp_path)
    failed = []
    for pin in P.ALL_PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, "no pin caught mutant %s" % name
    print("%s caught by %s" % (name, ", ".join(failed)))


def test_unmutated_copy_passes_every_pin(tmp_path):
    src = open(gemm_oracle.__file__).read()
    path = tmp_path / "gemm_copy.py"
    path.write_text(src)
    spec = importlib.util.spec_from_file_location("gemm_copy", str(path))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    for pin in P.ALL_PINS:
        pin(mod)
