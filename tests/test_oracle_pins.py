"""The oracle against its pins, and the pins against planted mistakes.

Every mutant below is a plausible slip in the oracle (wrong zero point, nibble
order, group index, dropped scale, swapped gate/up, eps placement, ...). It is
planted in a copy of the oracle source on the CPU, compiled with gcc, and must
fail at least one pin.
"""
import os

import pytest

import oracle
import oracle_pins as P

SRC = open(oracle.SRC).read()


@pytest.fixture(scope="module")
def o():
    return oracle.load()


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(o, pin):
    pin(o)


MUTANTS = P.MUTANTS


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_fails_some_pin(name, old, new):
    assert SRC.count(old) == 1, "mutation anchor must match exactly once: %r" % old
    bad = oracle.load_variant(SRC.replace(old, new), name)
    failed = []
    for pin in P.ALL_PINS:
        try:
            pin(bad)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, "mutant %s passed every pin" % name
