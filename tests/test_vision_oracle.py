"""The vision-block oracle against its pins, and planted mistakes in copies
of it that the pins must catch (CPU only)."""
import importlib.util

import pytest

import oracle
import pins_vision
from oracle import vision


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


@pytest.mark.parametrize("pin", pins_vision.ALL_PINS, ids=lambda p: p.__name__)
def test_vision_oracle_pin(pin, orc):
    pin(vision, orc)


MUTANTS = {
    "queries taken from the key block": ("qkv[:, 0 * hd:1 * hd]", "qkv[:, 1 * hd:2 * hd]"),
    "values taken from the key block": ("qkv[:, 2 * hd:3 * hd]", "qkv[:, 1 * hd:2 * hd]"),
    "heads strided instead of contiguous": (".reshape(T, H, d)", ".reshape(T, d, H).transpose(0, 2, 1)"),
    "attention output heads transposed": ("a.reshape(T, H * d)", "a.transpose(0, 2, 1).reshape(T, H * d)"),
    "QKV bias dropped": ("x @ w_qkv.T + b_qkv", "x @ w_qkv.T"),
    "output bias dropped": ("@ w_o.T + b_o", "@ w_o.T"),
    "mask ignored": ("cu_seqlens, mask, scale)", "cu_seqlens, 'full', scale)"),
    "scale ignored": ("mask, scale)", "mask, 1.0 / np.sqrt(d))"),
    "images merged": ("orc.attention(q, k, v, cu_seqlens,", "orc.attention(q, k, v, [0, T],"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_vision_planted_mistake_is_caught(name, orc, tmp_path):
    old, new = MUTANTS[name]
    src = open(vision.__file__).read()
    assert old in src, f"mutation site for {name!r} not found"
    path = tmp_path / "mutant_vision.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("mutant_vision", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    failed = []
    for pin in pins_vision.ALL_PINS:
        try:
            pin(mod, orc)
        except Exception:  # a wrong oracle may fail in any way
            failed.append(pin.__name__)
    assert failed, f"mutant {name!r} passed every pin"
