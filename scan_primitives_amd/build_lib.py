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


def compile_command(src: str, obj: str) -> list[str]:
    return [hipcc_path(), f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC", "-Wall", "-Wno-unused-function",
            "-I", INCLUDE, "-I", CSRC, *DEVICE_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]


def link_command(objs: list[str], out_path: str) -> list[str]:
    return [hipcc_path(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out_path, *objs]


def _run(cmd: list[str]) -> tuple[int, list[str]]:
    proc = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the device-only feature flag and says so; that is harmless.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    return proc.returncode, [ln for ln in (proc.stdout + proc.stderr).splitlines() if noise not in ln]


def build(verbose: bool = False) -> str:
    """Compile the library (always, even when one is already there) and return its path.

    Each source compiles to an object of its own, in parallel, under a build
    folder next to this file; then one link step writes the library."""
    from concurrent.futures import ThreadPoolExecutor

    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    jobs = [(src, os.path.join(objdir, os.path.splitext(src)[0] + ".o")) for src in SOURCES]
    cmds = [compile_command(src, obj) for src, obj in jobs]
    if verbose:
        for cmd in cmds:
            print(" ".join(cmd), flush=True)
    workers = max(1, min(len(cmds), os.cpu_count() or 1, 8))
    with ThreadPoolExecutor(max_workers=workers) as pool:
        results = list(pool.map(_run, cmds))
    errors = [(src, msgs) for (src, _), (rc, msgs) in zip(jobs, results) if rc != 0]
    if errors:
        raise RuntimeError("hipcc failed:\n" + "\n".join(f"{src}:\n" + "\n".join(msgs) for src, msgs in errors))
    if verbose:
        for (src, _), (_, msgs) in zip(jobs, results):
            if msgs:
                print("\n".join(msgs))
    tmp = LIB_PATH + ".tmp"
    rc, msgs = _run(link_command([obj for _, obj in jobs], tmp))
    if rc != 0:
        raise RuntimeError("hipcc link failed:\n" + "\n".join(msgs))
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


ASAN_LIB_PATH = os.path.join(HERE, "_build", "libsx_scan_asan.so")
# Host-side sanitizers for the C ABI layer (argument checks, planning, index maps).
# Each -fsanitize= sits behind -Xarch_host so that only host code is instrumented;
# the device objects are the ordinary ones.
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-shared-libasan"]


def asan_runtime() -> str:
    """Path of the clang AddressSanitizer runtime that a sanitized library needs preloaded."""
    import glob
    root = os.path.dirname(os.path.dirname(hipcc_path()))
    found = sorted(glob.glob(os.path.join(root, "llvm", "lib", "clang", "*", "lib", "linux",
                                          "libclang_rt.asan-x86_64.so")))
    if not found:
        raise RuntimeError("the AddressSanitizer runtime was not found beside hipcc")
    return found[-1]


def build_asan(verbose: bool = False) -> str:
    """A copy of the library whose host API layer (sx_api.cpp) runs under AddressSanitizer
    and UndefinedBehaviorSanitizer, linked with the ordinary device objects (built first
    if missing). Written under the build folder; returns its path."""
    objdir = os.path.join(HERE, "_build")
    objs = [os.path.join(objdir, os.path.splitext(src)[0] + ".o") for src in SOURCES if src != "sx_api.cpp"]
    if not all(os.path.exists(o) for o in objs):
        build(verbose)
    api_obj = os.path.join(objdir, "sx_api_asan.o")
    cmd = [hipcc_path(), f"--offload-arch={ARCH}", "-O1", "-g", "-std=c++20", "-fPIC", "-I", INCLUDE, "-I", CSRC,
           *DEVICE_FLAGS, *HOST_SANITIZE, "-c", os.path.join(CSRC, "sx_api.cpp"), "-o", api_obj]
    rc, msgs = _run(cmd)
    if rc != 0:
        raise RuntimeError("hipcc (sanitized sx_api.cpp) failed:\n" + "\n".join(msgs))
    rc, msgs = _run([hipcc_path(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *HOST_SANITIZE, "-o", ASAN_LIB_PATH,
                     api_obj, *objs])
    if rc != 0:
        raise RuntimeError("hipcc link (sanitized library) failed:\n" + "\n".join(msgs))
    return ASAN_LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
