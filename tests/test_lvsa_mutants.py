"""The LVSA pins must catch plausible mistakes in the LVSA oracle.

Each case plants one mistake in a copy of oracle/lvsa.py's source, loads it
as a module of its own and runs every pin of tests/test_lvsa_pins.py against
it: at least one has to fail.
"""
import os
import types

import pytest

import test_lvsa_pins as pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "lvsa.py")

MUTANTS = {
    "period_floor": ("return -(-T // (C - (2 * W + 1)))", "return max(1, T // (C - (2 * W + 1)))"),
    "globals_one_short": ("m = -(-T // T_per)\n    return sorted", "m = T // T_per\n    return sorted"),
    "globals_not_rotating": ("(s % T_per + i * T_per) % T", "(i * T_per) % T"),
    "window_lower_bound_unclamped": ("lo = max(0, min(t - W, T - 1 - 2 * W))", "lo = max(0, t - W)"),
    "window_too_narrow": ("return lo, min(T - 1, lo + 2 * W)", "return lo, min(T - 1, lo + 2 * W - 1)"),
    "no_expansion": ("while have < target:", "while False:"),
    "expansion_counts_globals": ("have = sum(1 for f in range(lo, hi + 1) if f not in gs)",
                                 "have = hi - lo + 1"),
    "tie_goes_later": ("if left >= right and left > 0:", "if left > right:"),
    "target_ignores_globals": ("target = min(2 * W + 1, T - len(gs))", "target = 2 * W + 1"),
    "no_softmax_scale": ("scale = 1.0 / math.sqrt(d)", "scale = 1.0"),
    "query_frame_off_by_one": ("keys = np.concatenate([np.arange(f * P, (f + 1) * P) for f in sets[t]])",
                               "keys = np.concatenate([np.arange(f * P, (f + 1) * P) for f in sets[min(t + 1, T - 1)]])"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, name
    mod = types.ModuleType("lvsa_mutant")
    exec(compile(src.replace(old, new), "lvsa_mutant.py", "exec"), mod.__dict__)
    monkeypatch.setattr(pins, "lvsa", mod)
    failed = []
    for fn in [getattr(pins, n) for n in dir(pins) if n.startswith("test_")]:
        try:
            fn()
        except (AssertionError, ValueError, IndexError, ZeroDivisionError):
            failed.append(fn.__name__)
    assert failed, "no pin caught mutant %s" % name
