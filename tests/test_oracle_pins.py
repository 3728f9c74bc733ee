"""The CPU oracle against facts fixed outside it (runs without a GPU)."""
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import oracle

from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_oracle_pin(pin):
    pin()


# Each deliberate mistake planted in the oracle (see orc_set_mutation in
# oracle/vbq_oracle.c) must make at least one pin fail.
MUTATIONS = {
    1: "dequantisation drops the offset",
    2: "dot product reads the wrong x index",
    3: "quantiser truncates instead of rounding",
    4: "canonical packing is MSB-first",
    5: "cell test uses > instead of >=",
    6: "residual added with the wrong sign",
    7: "scale divides by 2^b instead of 2^b - 1",
    8: "records of a class listed row-major instead of column-major",
    13: "compact in-cell fraction counted in 1/128 of the scale instead of 1/256",
    14: "compact in-cell encoding truncates instead of rounding to nearest",
    15: "compact in-cell decoding divides by 255 instead of 256",
    9: "record halves swapped",
    10: "bfloat16 rounding breaks ties away from zero",
    11: "re-quantisation drops the clamp to [0, L]",
    12: "re-quantisation takes L from the wrong width",
}


@pytest.mark.parametrize("m", sorted(MUTATIONS), ids=[MUTATIONS[m] for m in sorted(MUTATIONS)])
def test_oracle_mutation_is_caught(m):
    failed = []
    with oracle.mutation(m):
        for pin in ALL_PINS:
            if pin.__name__ == "pin_f16_conversion":
                continue
            try:
                pin()
            except AssertionError:
                failed.append(pin.__name__)
    assert failed, f"mutation {m} ({MUTATIONS[m]}) passed every pin"
