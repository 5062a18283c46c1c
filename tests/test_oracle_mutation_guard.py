"""Keeps the oracle's mutation check runnable and its hardest cases caught
(CPU only).

tests/oracle_mutations.py plants typical mistakes, one at a time, in a copy
of oracle/oracle.c and runs the oracle tests against each copy; it is run by
hand, since all of its mutations take about a minute.  This test is the part
that runs with the CPU suite: every mutation's text must still be found in
oracle.c (an edit of the oracle cannot leave the check silently unable to
plant a mistake), and the four mutations that once survived every pin (the
FP8 scale taken with a reciprocal, codes with a multiplier, combine's slot
order reversed and its FMA split into a multiply and an add) must still make
a test fail.
"""
import importlib.util
import os

import pytest

import oracle

_HERE = os.path.dirname(os.path.abspath(__file__))
_spec = importlib.util.spec_from_file_location("oracle_mutations",
                                               os.path.join(_HERE, "oracle_mutations.py"))
M = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(M)


def test_every_mutation_still_applies():
    with open(M.SRC) as f:
        src = f.read()
    names = set()
    for name, old, new, nth in M.MUTATIONS:
        assert name not in names, name
        names.add(name)
        assert old != new, name
        assert M.mutate(src, old, new, nth) != src, name


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", ["fp8_scale_by_reciprocal", "fp8_codes_by_multiplier",
                                  "combine_reversed_order", "combine_mul_then_add"])
def test_once_surviving_mutations_are_caught(name, tmp_path):
    m = next(m for m in M.MUTATIONS if m[0] == name)
    _, verdict, detail = M.run_one(m, list(oracle.GCC_FLAGS), str(tmp_path), False)
    assert verdict.startswith("caught"), (name, verdict, detail)
