"""The projection oracle against its pins, and planted mistakes in copies of
it that the pins must catch (CPU only)."""
import importlib.util
import os

import pytest

import pins_proj
from oracle import proj

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("pin", pins_proj.ALL_PINS, ids=lambda p: p.__name__)
def test_proj_oracle_pin(pin):
    pin(proj)


MUTANTS = {
    "scale along the input dim": ("scale[:, None]", "scale[None, :]"),
    "input dims reversed": ("return x @ w.T", "return x @ w[:, ::-1].T"),
    "rounding truncates": ("np.rint(m * 256.0)", "np.trunc(m * 256.0)"),
    "rounding ties away": ("np.rint(m * 256.0)", "np.floor(m * 256.0 + 0.5)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_proj_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(proj.__file__).read()
    assert old in src, f"mutation site for {name!r} not found"
    path = tmp_path / "mutant_proj.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("mutant_proj", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    failed = []
    for pin in pins_proj.ALL_PINS:
        try:
            pin(mod)
        except Exception:  # a wrong oracle may fail in any way
            failed.append(pin.__name__)
    assert failed, f"mutant {name!r} passed every pin"
