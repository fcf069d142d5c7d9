"""The GEMM comparators (oracle.gemm_check, oracle.gemm_check_f8) against planted results (no GPU),
and the pins' strength: each deliberately broken copy of the comparators must fail a pin."""
import importlib.util
import os

import pytest

import oracle
from tests import comparator_pins

ORACLE_INIT = os.path.join(os.path.dirname(os.path.abspath(oracle.__file__)), "__init__.py")


@pytest.mark.parametrize("pin", comparator_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_comparator_pin(pin):
    pin(oracle)


# (description, text in oracle/__init__.py, replacement)
MUTANTS = [
    ("finiteness test inverted into an escape", "ok = finite & (err <= bound)", "ok = finite | (err <= bound)"),
    ("strict comparison", "ok = finite & (err <= bound)", "ok = finite & (err < bound)"),
    ("bounds added instead of the larger taken", "bound = np.maximum(rtol * np.abs(r), atol)",
     "bound = rtol * np.abs(r) + atol"),
    ("smaller bound taken", "bound = np.maximum(rtol * np.abs(r), atol)", "bound = np.minimum(rtol * np.abs(r), atol)"),
    ("relative branch only", "bound = np.maximum(rtol * np.abs(r), atol)", "bound = rtol * np.abs(r)"),
    ("absolute branch only", "bound = np.maximum(rtol * np.abs(r), atol)", "bound = atol + 0 * r"),
    ("signed reference in the bound", "bound = np.maximum(rtol * np.abs(r), atol)", "bound = np.maximum(rtol * r, atol)"),
    ("signed error", "err = np.abs(g - r)", "err = g - r"),
    ("any instead of all", '"pass": bool(ok.all())', '"pass": bool(ok.any())'),
    ("shape check dropped", "    if g.shape != r.shape:\n        raise ValueError(f\"result shape",
     "    if False:\n        raise ValueError(f\"result shape"),
    ("relative tolerance ten times too wide", "rtol: float = 1e-2, atol: float = 1e-3,\n               extra",
     "rtol: float = 1e-1, atol: float = 1e-3,\n               extra"),
    ("absolute tolerance ten times too wide", "rtol: float = 1e-2, atol: float = 1e-3,\n               extra",
     "rtol: float = 1e-2, atol: float = 1e-2,\n               extra"),
    ("f8 widening dropped", "r = gemm_check(got, ref32, extra=dot_bound * absum)", "r = gemm_check(got, ref32)"),
    ("f8 signed dot instead of magnitudes", "a = np.abs(np.asarray(a_vals, dtype=np.float64))",
     "a = np.asarray(a_vals, dtype=np.float64)"),
    ("f8 B read as K×N", "absum = a @ b.T", "absum = a @ b"),
    ("f8 bound four times too wide", "F8_DOT_BOUND = 2.0 ** -13", "F8_DOT_BOUND = 2.0 ** -11"),
]


def _load_mutant(tmp_path, old, new):
    src = open(ORACLE_INIT).read()
    assert old in src, f"mutation site not found: {old!r}"
    path = tmp_path / "oracle_mutant.py"
    path.write_text(src.replace(old, new, 1))
    spec = importlib.util.spec_from_file_location("oracle_mutant", str(path))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)  # defines the comparators; the C oracle is not loaded
    return mod


@pytest.mark.parametrize("desc,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_broken_comparator_fails_a_pin(tmp_path, desc, old, new):
    mod = _load_mutant(tmp_path, old, new)
    failures = []
    for pin in comparator_pins.ALL_PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError, TypeError):
            failures.append(pin.__name__)
    assert failures, f"no pin catches: {desc}"
