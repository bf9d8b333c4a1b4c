"""Planted mistakes in the oracle (built on the CPU with -DORACLE_MUTANT=k)
must each fail at least one pin: the pins are strong enough to catch a
dropped term, a wrong sign, a wrong index or a transposed operand."""
import functools

import pytest

import oracle
from tests import pins

MUTANTS = {
    1: "D*x~ term dropped from y",
    2: "sign of the decay exponent flipped",
    3: "conv taps applied in reverse order",
    4: "parent's x~ used in the child's update",
    5: "y read from the parent state instead of the child state",
    6: "B and C swapped",
    7: "dt_bias dropped",
    8: "window rows read oldest-first past the root",
    9: "softplus replaced by exp",
    10: "commit forgets to shift the new token into the window",
    11: "validator accepts non-monotone parent[]",
    13: "commit applies the decay twice",
    14: "group of head h taken as h % G",
    15: "xbc: B channels convolved with the C channels' weights",
    16: "gate multiplies by sigmoid(z) instead of silu(z)",
    17: "xbc: commit shifts only x, not B and C, into the window",
    18: "bf16 state storage rounds ties up instead of to even",
    19: "path validator skips the root-level check of the first path node",
    20: "path validator's length bound off by one (rejects a full-length path)",
}

FAST_PINS = [pins.pin_chain_is_scan, pins.pin_closed_form, pins.pin_softplus_library, pins.pin_commit,
             pins.pin_validator, pins.pin_path_validator, functools.partial(pins.pin_bruteforce_forests, tmax=5), pins.pin_round_bf16]


@pytest.mark.parametrize("k", sorted(MUTANTS), ids=lambda k: "m%d" % k)
def test_mutant_is_caught(k):
    o = oracle.get(mutant=k)
    caught = []
    for pin in FAST_PINS:
        try:
            pin(o)
        except AssertionError:
            caught.append(getattr(pin, "__name__", getattr(getattr(pin, "func", None), "__name__", "?")))
    assert caught, "mutant %d (%s) passed every pin" % (k, MUTANTS[k])
