"""Plant mistakes in the oracle (on the CPU) and check that the pins catch
every one: a flipped kernel, a padding sign error, a dropped bias, a wrong
sign in the sigmoid, swapped kernel axes, a dropped input channel and an
off-by-one output size.  Each mutant is a separate gcc build of the oracle
source with -DCBS_ORACLE_MUTANT=k."""
import os

import pytest

import oracle
import oracle_pins

pytestmark = pytest.mark.cpu

MUTANTS = {1: "flipped kernel", 2: "pad sign", 3: "bias dropped", 4: "sigmoid sign",
           5: "kh/kw swapped", 6: "last channel dropped", 7: "output size off by one"}


@pytest.mark.parametrize("k", sorted(MUTANTS), ids=lambda k: MUTANTS[k].replace(" ", "_"))
def test_mutant_is_caught(k, tmp_path):
    path = oracle.build(os.path.join(tmp_path, f"mutant{k}.so"), mutant=k)
    bad = oracle.Oracle(path)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(bad)
        except Exception:  # an assertion or a shape error both count as a catch
            caught.append(pin.__name__)
    assert caught, f"no pin rejects mutant {k} ({MUTANTS[k]})"
