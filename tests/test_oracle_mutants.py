"""Planted mistakes in the oracle (on the CPU) must each fail some pin.

Each mutant is a copy of the oracle's C source with one plausible mistake
(a dropped term, a flipped sign, an off-by-one causal frontier, a swapped
operand, a missing scale), compiled to a temporary library.  Every pin in
``test_oracle_pins.py`` is run against it; at least one must fail.  This is
what makes the pins evidence that the oracle is right, rather than a retyping
of its formulas.
"""
import itertools
import os
import subprocess

import pytest

import oracle
from oracle import build_oracle
import test_oracle_pins as pins

MUTANTS = {
    "dS1 drops the -KL term": ("lp1 - lp2 - klv", "lp1 - lp2"),
    "dS2 sign flipped": ("g * (p2 - p1)", "g * (p1 - p2)"),
    "causal frontier one key short": ("int last = i + (n_k - n_q);", "int last = i + (n_k - n_q) - 1;"),
    "causal mask aligned top-left": ("int last = i + (n_k - n_q);", "int last = i;"),
    "dQ1 uses the student's keys": ("gq1[c] += scale * ds1 * kj1[c];", "gq1[c] += scale * ds1 * kj2[c];"),
    "dK2 misses the scale": ("gk2[c] += scale * ds2 * qi2[c];", "gk2[c] += ds2 * qi2[c];"),
    "KL weighted by P2": ("klv += exp(lp1) * (lp1 - lp2);", "klv += exp(lp2) * (lp1 - lp2);"),
    "LSE forgets the max": ("return m + log(s);", "return log(s);"),
    "S2 uses the teacher's keys": ("s2[j] = scale * dot(qi2, k2 +", "s2[j] = scale * dot(qi2, k1 +"),
    "dQ2 built from queries": ("gq2[c] += scale * ds2 * kj2[c];", "gq2[c] += scale * ds2 * qi2[c];"),
    "dK1 sums the student's queries": ("gk1[c] += scale * ds1 * qi1[c];", "gk1[c] += scale * ds1 * qi2[c];"),
    "LSE1 from the student": ("const double L1 = logsumexp(s1, nj);", "const double L1 = logsumexp(s2, nj);"),
}


def _pin_cases():
    """Every (test function, kwargs) of the pin module, parametrisations expanded."""
    cases = []
    for name in sorted(dir(pins)):
        fn = getattr(pins, name)
        if not (name.startswith("test_") and callable(fn)):
            continue
        marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        grids = []
        for m in marks:
            argnames = [a.strip() for a in m.args[0].split(",")] if isinstance(m.args[0], str) else list(m.args[0])
            vals = [v if len(argnames) > 1 else (v,) for v in m.args[1]]
            grids.append([dict(zip(argnames, v)) for v in vals])
        for combo in itertools.product(*grids) if grids else [()]:
            kw = {}
            for part in combo:
                kw.update(part)
            cases.append((name, fn, kw))
    return cases


@pytest.fixture(scope="module")
def source():
    with open(build_oracle.SRC) as f:
        return f.read()


@pytest.mark.parametrize("label", sorted(MUTANTS))
def test_mutant_is_caught(label, source, tmp_path, monkeypatch):
    old, new = MUTANTS[label]
    assert source.count(old) == 1, f"mutation anchor not unique: {old!r}"
    src = tmp_path / "mutant.c"
    src.write_text(source.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                    str(src), "-o", str(lib), "-lm"], check=True)
    monkeypatch.setattr(oracle, "_lib", oracle.load_library(str(lib)))
    caught = []
    for name, fn, kw in _pin_cases():
        try:
            fn(**kw)
        except AssertionError:
            caught.append(name)
    assert caught, f"no pin catches the mutant '{label}'"


def test_unmutated_oracle_passes_every_pin():
    for name, fn, kw in _pin_cases():
        fn(**kw)
