"""The oracle's pins catch plausible mistakes: each case plants one slip in a
copy of oracle.cpp (a dropped term, a wrong index, swapped operands), builds
that copy into a temporary library, and checks that at least one pin fails
against it while all pass against the real oracle."""
import ctypes
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.cpp")

# (what, text in oracle.cpp, replacement, pins expected to catch it)
MUTANTS = [
    ("routed term dropped", "y[r] = up[r] + sh[r];", "y[r] = sh[r];",
     ["test_output_at_the_situ_caps_is_exact",
      "test_output_without_shared_experts_selects_latent_entries"]),
    ("shared sum dropped", "y[r] = up[r] + sh[r];", "y[r] = up[r];",
     ["test_output_at_the_situ_caps_is_exact"]),
    ("only the first shared expert", "for (int64_t j = 0; j < s->n_shared; ++j) {",
     "for (int64_t j = 0; j < 1; ++j) {", ["test_output_at_the_situ_caps_is_exact"]),
    ("gate and up swapped in the shared experts",
     "for (int64_t i = 0; i < Is; ++i) h[i] = orc_phi(g[i], s->beta) * orc_psi(u[i], s->beta_u);",
     "for (int64_t i = 0; i < Is; ++i) h[i] = orc_phi(u[i], s->beta) * orc_psi(g[i], s->beta_u);",
     ["test_output_at_the_situ_caps_is_exact"]),
    ("shared down matrix of the wrong expert",
     "orc_matvec(&w->sh_down, j, h.data(), part.data());",
     "orc_matvec(&w->sh_down, 0, h.data(), part.data());",
     ["test_output_at_the_situ_caps_is_exact"]),
]


def _build(tmp_path, text):
    src = tmp_path / "oracle_mutant.cpp"
    src.write_text(text)
    lib = tmp_path / "liboracle_mutant.so"
    subprocess.run(["g++", "-O1", "-std=c++17", "-fPIC", "-shared", "-fopenmp",
                    "-ffp-contract=off", "-I", os.path.dirname(SRC), "-o", str(lib), str(src)],
                   check=True)
    return str(lib)


def _fails(name):
    try:
        getattr(pins, name)()
    except AssertionError:
        return True
    return False


@pytest.mark.parametrize("what,old,new,caught_by", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, what, old, new, caught_by):
    text = open(SRC).read()
    assert text.count(old) >= 1, f"mutation site missing: {old}"
    for name in caught_by:  # the real oracle passes
        assert not _fails(name), name
    path = _build(tmp_path, text.replace(old, new, 1))
    saved = oracle._lib
    try:
        oracle._lib = None
        real_cdll = ctypes.CDLL
        # load the mutant in place of liboracle.so for this test only
        ctypes.CDLL = lambda p, *a, **k: real_cdll(path if p.endswith("liboracle.so") else p,
                                                   *a, **k)
        oracle.lib()
    finally:
        ctypes.CDLL = real_cdll
    try:
        caught = [n for n in caught_by if _fails(n)]
    finally:
        oracle._lib = saved
    assert caught, f"no pin catches: {what}"
