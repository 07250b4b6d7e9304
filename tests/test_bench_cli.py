"""bench.py's command-line contract that holds without a GPU: one GPU only
(--gpus above 1 exits with status 2 and says why, before touching a device),
and the headline summaries it reads from profiles/ parse and name the kernel
source digest they were taken on (the bench reports their traffic and
counters only while that digest matches the sources, else null)."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_profile_summaries_parse():
    b = _bench_module()
    for path in (b.TRAFFIC_FILE, b.COUNTERS_FILE):
        fields = {}
        with open(path) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    fields[k.strip()] = v.strip()
        assert len(fields.get("kernel_source_sha256_16", "")) == 16, path

