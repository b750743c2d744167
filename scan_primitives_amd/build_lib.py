"""Build libsx_scan.so in-tree with hipcc for gfx950.

Run as ``python -m scan_primitives_amd.build_lib``; ``__graft_entry__.build()``
calls :func:`build` as well. The library is written next to this file so that
it travels with the source tree.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libsx_scan.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

SOURCES = ["sx_api.cpp", "element_scan.hip", "normcap_quad.hip", "matrix_scan.hip", "matrix_scan_grad.hip",
           "table_scan.hip"]
ARCH = "gfx950"

# Packed FP32 (v_pk_*_f32) stays off for all device code: the kernels are
# written for scalar f32 VALU and MFMA only.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc_path() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def build_command(out_path: str = LIB_PATH) -> list[str]:
    cmd = [hipcc_path(), f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-shared", "-fPIC",
           "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC, *DEVICE_FLAGS, "-o", out_path]
    cmd += [os.path.join(CSRC, s) for s in SOURCES]
    return cmd


def build(verbose: bool = False) -> str:
    """Compile the library (always, even when one is already there) and return its path."""
    tmp = LIB_PATH + ".tmp"
    cmd = build_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the device-only feature flag and says so; that is harmless.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = [ln for ln in (proc.stdout + proc.stderr).splitlines() if noise not in ln]
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
