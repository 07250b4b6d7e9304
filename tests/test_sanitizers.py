"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

Builds, with -fsanitize=address,undefined (errors fatal): the two C oracles,
and the library's host-only units (the C ABI's argument checks and work
planning: attn_api.cpp, gdn_api.cpp, vision_api.cpp, proj_api.cpp) linked
with stand-ins for the device entry points (tests/host_stubs.cpp).  Then runs
the oracle pin tests and the ABI-check tests against those builds in a child
process with the sanitizer runtime preloaded.  No GPU code is built or run.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_attention_prefill_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g",
       "-O1"]
HOST_UNITS = ("attn_api.cpp", "gdn_api.cpp", "vision_api.cpp", "proj_api.cpp")
TESTS = ("test_abi.py", "test_gdn_abi.py", "test_vision_abi.py", "test_proj_abi.py", "test_oracle.py",
         "test_gdn_oracle.py", "test_proj_oracle.py", "test_vision_oracle.py", "test_probes_cpu.py")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


@pytest.fixture(scope="module")
def san_builds(tmp_path_factory):
    if shutil.which("gcc") is None or shutil.which("g++") is None:
        pytest.skip("gcc/g++ not available")
    out = tmp_path_factory.mktemp("san")
    libs = {}
    for name, src in (("attn", "attn_oracle.c"), ("gdn", "gdn_oracle.c")):
        lib = str(out / f"lib{name}_oracle_san.so")
        _run(["gcc", *SAN, "-fopenmp", "-fPIC", "-shared", "-o", lib, os.path.join(ROOT, "oracle", src),
              "-lm"])
        libs[name] = lib
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC, "-isystem", os.path.join(ROCM, "include"),
           "-D__HIP_PLATFORM_AMD__"]
    objs = []
    for src in (*[os.path.join(CSRC, u) for u in HOST_UNITS], os.path.join(ROOT, "tests", "host_stubs.cpp")):
        obj = str(out / (os.path.basename(src) + ".o"))
        _run(["g++", *SAN, "-std=c++17", "-fPIC", "-Wall", *inc, "-c", src, "-o", obj])
        objs.append(obj)
    host = str(out / "libattn_prefill_host_san.so")
    _run(["g++", *SAN, "-shared", "-o", host, *objs, "-L" + os.path.join(ROCM, "lib"), "-lhipblaslt",
          "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")])
    libs["host"] = host
    return libs


def test_host_code_under_sanitizers(san_builds):
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    assert os.path.isabs(asan) and os.path.exists(asan), "libasan not found"
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": asan,
        # the interpreter and torch keep allocations alive at exit by design
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "ATTN_PREFILL_LIBRARY": san_builds["host"],
        "ATTN_ORACLE_LIBRARY": san_builds["attn"],
        "GDN_ORACLE_LIBRARY": san_builds["gdn"],
        "OMP_NUM_THREADS": "4",
    })
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
           *[os.path.join(ROOT, "tests", t) for t in TESTS]]
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, cwd=ROOT, timeout=900)
    report = r.stdout[-6000:] + r.stderr[-6000:]
    assert r.returncode == 0, report
    assert "ERROR: AddressSanitizer" not in report and "runtime error:" not in report, report
    assert " passed" in r.stdout, report


def test_sanitizer_setup_catches_a_heap_overflow(tmp_path):
    """The same flags, preload and options stop a child that reads past a heap
    block: the check above is not vacuous."""
    src = tmp_path / "oob.c"
    src.write_text("#include <stdlib.h>\n"
                   "int oob(int n) { int *p = malloc(4 * sizeof(int)); for (int i = 0; i < 4; ++i) p[i] = i;\n"
                   "  int x = p[n]; free(p); return x; }\n")
    lib = str(tmp_path / "liboob.so")
    _run(["gcc", *SAN, "-fPIC", "-shared", "-o", lib, str(src)])
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    code = f"import ctypes; l = ctypes.CDLL({lib!r}); print(l.oob(1)); print(l.oob(4))"
    r = subprocess.run([sys.executable, "-u", "-c", code], capture_output=True, text=True, env=env, timeout=120)
    # UndefinedBehaviorSanitizer (object-size check) or AddressSanitizer stops it
    caught = "heap-buffer-overflow" in r.stderr or "runtime error:" in r.stderr
    assert r.returncode != 0 and caught, r.stderr[-2000:]
    assert r.stdout.strip().splitlines()[0] == "1"
