"""Planted mistakes in the oracle must each trip at least one pin.

Each mutant is a textual change to a copy of oracle/attn_oracle.c (a dropped
term, a wrong sign or index, a swapped operand), compiled with gcc into a
temporary directory and run through every pin in a process of its own, so a
mutant that crashes is reported as caught rather than taking pytest down.
"""
import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))

MUTANTS = {
    "causal drops the diagonal": ("*hi = i + 1;", "*hi = i;"),
    "causal sees one key ahead": ("*hi = i + 1;", "*hi = i + 2 < n ? i + 2 : n;"),
    "window one short": ("int64_t end = start + window;", "int64_t end = start + window - 1;"),
    "window misaligned": ("int64_t start = (i / window) * window;",
                          "int64_t start = (i / window) * window + (i / window > 0);"),
    "full mask drops last key": ("*hi = n;\n    } else {", "*hi = n - 1;\n    } else {"),
    "gqa maps by modulo": ("int g = h / (hq / hkv);", "int g = h % hkv;"),
    "scale dropped": ("scores[j - lo] = scale * dot;", "scores[j - lo] = dot;"),
    "exponent sign flipped": ("exp(scores[j - lo] - m)", "exp(m - scores[j - lo])"),
    "max not subtracted": ("exp(scores[j - lo] - m)", "exp(scores[j - lo])"),
    "scores use V": ("const double *kj = kseq + ", "const double *kj = vseq + "),
    "key sequence offset dropped": ("k + (size_t)cu_k[b] * hkv * d;", "k;"),
    "value head ignored": ("vseq + ((size_t)j * hkv + g) * d", "vseq + ((size_t)j * hkv) * d"),
    "query head ignored": ("q + ((size_t)t * hq + h) * d", "q + ((size_t)t * hq) * d"),
    "normalisation dropped": ("double p = scores[j - lo] / l;", "double p = scores[j - lo];"),
    "sequence lookup off by one": ("(int64_t)cu[b + 1] <= t", "(int64_t)cu[b + 1] < t"),
    "lse drops the max": ("*lse = m + log(l);", "*lse = log(l);"),
    "queries aligned top-left": ("int64_t pos = (t - cu_q[b]) + (lk - lq);",
                                 "int64_t pos = (t - cu_q[b]);"),
    "key count from the query packing": ("int64_t lk = (int64_t)cu_k[b + 1] - cu_k[b];",
                                         "int64_t lk = (int64_t)cu_q[b + 1] - cu_q[b];"),
    "values from the query packing": ("v + (size_t)cu_k[b] * hkv * d;", "v + (size_t)cu_q[b] * hkv * d;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle.SOURCE).read()
    assert old in src, f"mutation site for {name!r} not found"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new, 1))
    lib = str(tmp_path / "libmutant.so")
    oracle.build(str(mutated), lib)
    proc = subprocess.run([sys.executable, os.path.join(HERE, "run_pins.py"), lib, "--first"],
                          capture_output=True, text=True, timeout=600)
    lines = proc.stdout.splitlines()
    caught = proc.returncode != 0 or any(l.startswith("FAIL") for l in lines)
    assert caught, f"mutant {name!r} passed every pin:\n" + proc.stdout
