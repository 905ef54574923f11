"""Run every oracle pin against one oracle library (used for planted-mistake copies).

Exit status 0: some pin failed (the planted mistake was caught); 3: every pin passed."""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import pins  # noqa: E402
from oracle import oracle as O  # noqa: E402

lib = O.load(sys.argv[1])
# the pins of the mutated routine's family first (only the time to the first failure changes)
family = {"q": "pin_q", "conv": "pin_conv"}.get((sys.argv[2] if len(sys.argv) > 2 else "").split("_")[0], "")
order = sorted(pins.ALL_PINS, key=lambda p: (not (family and p.__name__.startswith(family)) and
                                             not (family == "pin_q" and p.__name__ == "pin_requantize_definition"),
                                             p is pins.pin_brute_force_gather))
for pin in order:
    try:
        pin(lib)
    except (AssertionError, O.OracleError) as e:
        print(f"caught by {pin.__name__}: {str(e)[:200]}")
        sys.exit(0)
print("not caught")
sys.exit(3)
