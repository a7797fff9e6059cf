"""Each planted mistake in the oracle is caught by at least one pin (CPU only).

The oracle source compiles one deliberate error when built with
-DPKV_ORACLE_PLANT=n; the default build has none.
"""
import pytest

import oracle as O
from pins import ATTENTION_PINS

PLANTS = {
    1: "drops the newest key",
    2: "interleaved instead of contiguous head groups",
    3: "softmax scale dropped",
    4: "page index off by one token",
    5: "K rows read in place of V rows",
}


@pytest.mark.parametrize("plant", sorted(PLANTS), ids=lambda p: PLANTS[p].replace(" ", "_"))
def test_plant_is_caught(plant):
    orc = O.Oracle(plant)
    assert orc.lib.pkv_oracle_plant() == plant
    caught = []
    for pin in ATTENTION_PINS:
        try:
            pin(orc)
        except (AssertionError, O.OracleError) as e:
            caught.append((pin.__name__, str(e)[:80]))
    assert caught, f"planted mistake '{PLANTS[plant]}' passed every pin"


def test_clean_build_has_no_plant():
    assert O.Oracle(0).lib.pkv_oracle_plant() == 0
