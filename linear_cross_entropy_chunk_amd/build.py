"""Build liblce.so for gfx950 in-tree with hipcc (no GPU needed).

    python -m linear_cross_entropy_chunk_amd.build

Each translation unit under csrc/ is compiled in parallel into _build/ at the
repository root, then linked into linear_cross_entropy_chunk_amd/liblce.so.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG_DIR, "liblce.so")
SOURCES = ["lce_gemm.hip", "lce_rowops.hip", "lce_api.hip"]

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-fvisibility=hidden",
    # No packed-fp32 VALU instructions in device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _run(cmd: list[str]) -> None:
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    if out.strip():
        print(out, file=sys.stderr)


def build(verbose: bool = True) -> str:
    """Compile every HIP source and link liblce.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([HIPCC, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(len(cmds)) as ex:
        list(ex.map(_run, cmds))
    tmp = LIB_PATH + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    build_c_client(verbose)
    return LIB_PATH


C_CLIENT_SRC = os.path.join(ROOT, "tests", "c_abi", "lce_client.c")
C_CLIENT = os.path.join(ROOT, "tests", "c_abi", "lce_client")


def build_c_client(verbose: bool = True) -> str | None:
    """The plain C client the GPU tests use to call liblce.so without
    PyTorch (host code only; it finds the library through its rpath)."""
    if not os.path.exists(C_CLIENT_SRC):
        return None
    rpath = "$ORIGIN/" + os.path.relpath(PKG_DIR, os.path.dirname(C_CLIENT))
    rocm = os.environ.get("ROCM_PATH") or os.path.dirname(os.path.dirname(
        os.path.realpath(HIPCC)))
    tmp = C_CLIENT + ".tmp"
    _run([HIPCC, "-O2", "-std=c11", "-Wall", "-D__HIP_PLATFORM_AMD__",
          "-I", os.path.join(ROOT, "include"), "-I", os.path.join(rocm, "include"),
          C_CLIENT_SRC, "-o", tmp, "-L", PKG_DIR, "-llce", "-L", os.path.join(rocm, "lib"),
          "-lamdhip64", f"-Wl,-rpath,{rpath}"])
    os.replace(tmp, C_CLIENT)
    if verbose:
        print(f"built {C_CLIENT}")
    return C_CLIENT


if __name__ == "__main__":
    build()
