"""The STA pins must catch plausible mistakes in the STA oracle: each case
plants one mistake in a copy of oracle/sta.py's source, loads it as a module
of its own and runs every pin of tests/test_sta_pins.py against it."""
import os
import types

import pytest

import test_sta_pins as pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "sta.py")

MUTANTS = {
    "centre_floor_half": ("(np.asarray(i) // t) * t + (t + 1) // 2", "(np.asarray(i) // t) * t + t // 2"),
    "closed_on_the_left": ("return (2 * d > -W) & (2 * d <= W)", "return (2 * d >= -W) & (2 * d <= W)"),
    "open_on_the_right": ("return (2 * d > -W) & (2 * d <= W)", "return (2 * d > -W) & (2 * d < W)"),
    "full_window_as_half": ("return (2 * d > -W) & (2 * d <= W)", "return (d > -W) & (d <= W)"),
    "token_not_tile_centre": ("d = centre(j, t) - centre(i, t)", "d = np.asarray(j) - centre(i, t)"),
    "axes_or_not_and": ("        keep &= axis_keep(c[:, a][:, None], c[:, a][None, :], tile[a], window[a])",
                        "        keep = keep & axis_keep(c[:, a][:, None], c[:, a][None, :], tile[a], window[a]) if a == 0 else keep | axis_keep(c[:, a][:, None], c[:, a][None, :], tile[a], window[a])"),
    "tile_order_inner_transposed": ("inner = ((c[:, 0] % tf) * th + c[:, 1] % th) * tw + c[:, 2] % tw",
                                    "inner = ((c[:, 2] % tw) * th + c[:, 1] % th) * tf + c[:, 0] % tf"),
    "no_softmax_scale": ("scale = 1.0 / math.sqrt(d)", "scale = 1.0"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, name
    mod = types.ModuleType("sta_mutant")
    exec(compile(src.replace(old, new), "sta_mutant.py", "exec"), mod.__dict__)
    monkeypatch.setattr(pins, "sta", mod)
    failed = []
    for fn in [getattr(pins, n) for n in dir(pins) if n.startswith("test_")]:
        try:
            fn()
        except (AssertionError, ValueError, IndexError, ZeroDivisionError):
            failed.append(fn.__name__)
    assert failed, "no pin caught mutant %s" % name
