"""The fp64 gated-delta-rule oracle against its pins, and planted mistakes in
copies of its source that the pins must catch (CPU only)."""
import os
import subprocess
import sys

import numpy as np
import pytest

import pins_gdn
from oracle import gdn

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def gdn_orc():
    return gdn.load()


@pytest.mark.parametrize("pin", pins_gdn.ALL_PINS, ids=lambda p: p.__name__)
def test_gdn_oracle_pin(gdn_orc, pin):
    pin(gdn_orc)


def test_gdn_oracle_rejects_bad_arguments(gdn_orc):
    q = np.zeros((4, 2, 8))
    v = np.zeros((4, 2, 3))
    g = np.zeros((4, 2))
    with pytest.raises(ValueError):
        gdn_orc.gated_delta_rule(q, q, v, g, g, [0, 3], 1.0)
    with pytest.raises(ValueError):
        gdn_orc.gated_delta_rule(q, q, v, g, g, [0, 3, 2, 4], 1.0)
    with pytest.raises(ValueError):
        gdn_orc.gated_delta_rule(q, q, v, np.zeros((4, 1)), g, [0, 4], 1.0)
    with pytest.raises(ValueError):
        gdn_orc.gated_delta_rule(q, q, v, g, g, [0, 4], 1.0, initial_state=np.zeros((1, 2, 8, 3)))


MUTANTS = {
    "decay dropped": ("S[i] *= alpha;", "S[i] *= 1.0;"),
    "beta dropped on the write": ("u[i] = bt * (vt[i] - sk);", "u[i] = (vt[i] - sk);"),
    "no delta correction": ("u[i] = bt * (vt[i] - sk);", "u[i] = bt * vt[i];"),
    "correction sign flipped": ("u[i] = bt * (vt[i] - sk);", "u[i] = bt * (vt[i] + sk);"),
    "state transposed on read": ("acc += S[(size_t)i * dk + j] * (scale * qt[j]);",
                                 "acc += S[(size_t)j * dv + i] * (scale * qt[j]);"),
    "output read before the write": ("acc += S[(size_t)i * dk + j] * (scale * qt[j]);",
                                     "acc += (S[(size_t)i * dk + j] - u[i] * kt[j]) * (scale * qt[j]);"),
    "gate of the previous token": ("const double alpha = exp(g[th])",
                                   "const double alpha = exp(g[th >= (size_t)h ? th - h : th])"),
    "scale dropped": ("(scale * qt[j])", "(qt[j])"),
    "initial state ignored": ("if (s0 != NULL)\n", "if (0)\n"),
    "value head ignored": ("*vt = v + th * dv;", "*vt = v + (size_t)t * h * dv;"),
    "key used as query": ("*qt = q + th * dk,", "*qt = k + th * dk,"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_gdn_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(gdn.SOURCE).read()
    assert old in src, f"mutation site for {name!r} not found"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new, 1))
    lib = str(tmp_path / "libmutant.so")
    gdn.build(str(mutated), lib)
    proc = subprocess.run([sys.executable, os.path.join(HERE, "run_gdn_pins.py"), lib, "--first"],
                          capture_output=True, text=True, timeout=600)
    lines = proc.stdout.splitlines()
    caught = proc.returncode != 0 or any(l.startswith("FAIL") for l in lines)
    assert caught, f"mutant {name!r} passed every pin:\n" + proc.stdout
