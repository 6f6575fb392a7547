"""Build the HIP library in-tree: decode_attention_head_amd/libdah.so (gfx950).

    python -m decode_attention_head_amd.build

Every call recompiles.  The library is one shared object with a plain C ABI
(include/dah.h); nothing is JIT-compiled at import time.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libdah.so")
PROBE_LIB_PATH = os.path.join(PKG_DIR, "libdah_probe.so")

# (output, sources): the attention library and the benchmark's memory probes
TARGETS = [
    (LIB_PATH, ["dah_kernels.hip", "dah_linear.hip", "dah_layer.hip", "dah_host.cpp"]),
    (PROBE_LIB_PATH, ["dah_probe.hip"]),
]

# Packed FP32 instructions are disabled for all device code (the compiler
# would otherwise form v_pk_* from float code).
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Werror=return-type",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _compile(out: str, sources: list, verbose: bool) -> None:
    cmd = [hipcc(), *HIP_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}",
           *[os.path.join(CSRC, s) for s in sources], "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if msgs and verbose:
        print("\n".join(msgs))
    os.replace(out + ".tmp", out)


def build(verbose: bool = False) -> str:
    for out, sources in TARGETS:
        _compile(out, sources, verbose)
    return LIB_PATH


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
