"""Mutation test of the oracle's pins.

Each build with -DORACLE_MUTATION=k plants one plausible mistake in the CPU
oracle (on the CPU only): a dropped diagonal, a reversed bit order, a wrong sign
in the Gray update, a missing field update, a traversal-order tie-break, a
count that ignores ties, a field without its diagonal, a dropped x_j factor,
a flip applied to the wrong variable, an off-by-one in the k-lowest list, a
floating-point sum in the wrong order, floating-point ties within a tolerance
and floating-point k-lowest lists merged without the index order of ties.
The pin suite must reject every one.
"""
import pytest

import oracle
from test_oracle_pins import ALL_PINS, ALL_PINS_F64

MUTANTS = {
    1: "energy drops the diagonal terms",
    2: "energy reads variable i from bit i (LSB first)",
    3: "Gray walk adds the field on a 1->0 flip",
    4: "Gray walk never updates the fields",
    5: "ties keep the first state met in traversal order",
    6: "ties are not counted",
    7: "initial fields miss the diagonal",
    8: "energy drops the x_j factor",
    9: "Gray walk flips variable t instead of n-1-t",
    10: "the k-lowest list never fills its last slot after it is full",
    11: "floating-point energies summed in column-major order",
    12: "floating-point energies within a relative 1e-12 count as ties",
    13: "the floating-point k-lowest lists merge last thread first, equal energies in the order met",
}


@pytest.mark.parametrize("k", sorted(MUTANTS))
def test_pins_reject_mutant(k, tmp_path):
    path = oracle.build(str(tmp_path / ("liboracle_m%d.so" % k)), defines=("ORACLE_MUTATION=%d" % k,))
    o = oracle.Oracle(path)
    failed = []
    for pin in ALL_PINS + ALL_PINS_F64:
        try:
            pin(o)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, "mutant %d (%s) passed every pin" % (k, MUTANTS[k])
