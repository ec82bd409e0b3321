"""The CPU oracle pinned against closed forms, library conversions, exact
rational arithmetic and the method's invariants (see pins.py)."""
import json
import os

import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def L():
    # test_sanitizers.py reruns the pins on a -fsanitize=address,undefined
    # build of fp8_oracle.c, named by ORACLE_LIB
    if os.environ.get("ORACLE_LIB"):
        return oracle.OracleLib(os.environ["ORACLE_LIB"])
    oracle.build(force=False)
    return oracle.default()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(L, pin):
    pin(L)


def test_fpu_is_ieee(L):
    assert L.L.oracle_fpu_check() == 0


def test_stored_zero_constants_match_exact_math():
    with open(os.path.join(pins.GOLDEN, "zero_and_empty_constants.json")) as f:
        stored = json.load(f)
    derived = pins.zero_constants_from_math()
    assert stored["clamp_1e-4"] == derived["clamp_1e-4"]
    for fmt in pins.FORMATS:
        for k, v in derived[fmt].items():
            assert stored[fmt][k] == v, (fmt, k)
