"""Build the HIP library in-tree: ``python -m long_context_attention_prefill_amd.build``.

Produces ``long_context_attention_prefill_amd/libattn_prefill.so`` for gfx950:
the kernels (csrc/*.hip) compiled by hipcc, the host-only C ABI
(csrc/*_api.cpp) compiled by g++, linked by hipcc against hipBLASLt (the
vendor GEMM of the projections).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
LIBRARY = os.path.join(PKG, "libattn_prefill.so")
ARCH = "gfx950"

# Kernel sources: attention prefill (both families), decode, gated delta rule,
# projections (int8 dequantization).
DEVICE_SOURCES = ("attn_fwd.hip", "attn_decode.hip", "gdn_fwd.hip", "proj_fwd.hip")
# Host-only sources (C ABI: checks and planning), compiled by g++.
HOST_SOURCES = ("attn_api.cpp", "gdn_api.cpp", "proj_api.cpp", "vision_api.cpp")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
# the projections call the vendor GEMM (hipBLASLt)
LINK_LIBS = ["-L" + os.path.join(ROCM, "lib"), "-lhipblaslt"]

# Packed-fp32 VALU forms are kept out of every kernel on purpose.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose: bool = False, output: str = LIBRARY, extra_device_flags=()) -> str:
    hipcc = _hipcc()
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    with tempfile.TemporaryDirectory() as tmp:
        objs = []
        for src in HOST_SOURCES:
            obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
            _run(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", *inc,
                  "-isystem", os.path.join(ROCM, "include"), "-D__HIP_PLATFORM_AMD__", "-c",
                  os.path.join(CSRC, src), "-o", obj], verbose)
            objs.append(obj)
        for src in DEVICE_SOURCES:
            obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
            _run([hipcc, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", *DEVICE_FLAGS,
                  *extra_device_flags, *inc, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
            objs.append(obj)
        tmp_out = output + ".tmp"
        _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp_out, *objs, *LINK_LIBS,
              "-Wl,-rpath," + os.path.join(ROCM, "lib")], verbose)
        os.replace(tmp_out, output)
    return output


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
