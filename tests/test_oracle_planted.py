"""Plant plausible mistakes in the oracle (separate CPU builds) and check the pins catch each one."""
import pytest

import oracle
from oracle_pins import ALL_PINS

# planted mistake id -> (what it is, pins that must fail)
PLANTED = {
    1: ("softmax scale dropped", {"pin_brute_force_dense", "pin_brute_force_paged", "pin_single_key"}),
    2: ("value taken from the last 512 dims", {"pin_brute_force_paged", "pin_single_key"}),
    3: ("wrong sign in the max subtraction", {"pin_dominant_key"}),
    4: ("base-2 log in the LSE", {"pin_brute_force_dense", "pin_zero_query"}),
    5: ("K read transposed", {"pin_brute_force_dense", "pin_transposed_identity"}),
    6: ("off-by-one causal visibility", {"pin_brute_force_paged", "pin_causal_rows"}),
    7: ("pages assumed contiguous", {"pin_brute_force_paged", "pin_page_relabelling"}),
}


@pytest.mark.parametrize("mistake", sorted(PLANTED), ids=[PLANTED[k][0] for k in sorted(PLANTED)])
def test_planted_mistake_is_caught(mistake):
    orc = oracle.Oracle(planted_mistake=mistake)
    failed = set()
    for pin in ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, RuntimeError, ValueError, FloatingPointError):
            failed.add(pin.__name__)
    missing = PLANTED[mistake][1] - failed
    assert not missing, f"planted mistake {mistake} ({PLANTED[mistake][0]}) not caught by {missing}; failed: {failed}"
