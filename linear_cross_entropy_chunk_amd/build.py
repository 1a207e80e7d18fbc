"""Build liblce.so for gfx950 in-tree with hipcc (no GPU needed).

    python -m linear_cross_entropy_chunk_amd.build [--sanitize]

Each translation unit under csrc/ is compiled in parallel into _build/ at the
repository root, then linked into linear_cross_entropy_chunk_amd/liblce.so.

With sanitize=True it also builds tests/c_abi/lce_host_checks: the C ABI's
host code (planner, validation, workspace layout) compiled for the host only
under AddressSanitizer and UndefinedBehaviorSanitizer, linked with a C
harness that walks valid and invalid problem descriptions.  It runs on the
CPU and launches no kernel.
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


def build(verbose: bool = True, sanitize: bool = False) -> str:
    """Compile every HIP source and link liblce.so; returns the library path.
    sanitize=True also builds the sanitized host-check program."""
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
    if sanitize:
        build_host_checks(verbose)
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


HOST_CHECKS_SRC = os.path.join(ROOT, "tests", "c_abi", "lce_host_checks.c")
HOST_CHECKS = os.path.join(ROOT, "tests", "c_abi", "lce_host_checks")
SAN_DIR = os.path.join(BUILD_DIR, "sanitize")
# Host-only sanitizer flags.  On the hipcc line each -fsanitize= comes right
# after -Xarch_host, so the device code is built without them; the plain
# clang lines below name no HIP source.
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_C = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
         "-fno-omit-frame-pointer"]


def _rocm() -> str:
    return os.environ.get("ROCM_PATH") or os.path.dirname(os.path.dirname(
        os.path.realpath(HIPCC)))


def build_host_checks(verbose: bool = True) -> str:
    """The C ABI's host code under ASan + UBSan, linked with the C harness
    tests/c_abi/lce_host_checks.c into one CPU program.  The kernels' objects
    are linked as built for liblce.so (their host-side launchers are never
    reached: every call the harness makes fails validation first)."""
    os.makedirs(SAN_DIR, exist_ok=True)
    objs = [os.path.join(BUILD_DIR, s.replace(".hip", ".o")) for s in SOURCES if s != "lce_api.hip"]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        build(verbose=False)
    rocm = _rocm()
    clang = os.path.join(rocm, "llvm", "bin", "clang")
    api_o = os.path.join(SAN_DIR, "lce_api_host.o")
    harness_o = os.path.join(SAN_DIR, "lce_host_checks.o")
    _run([HIPCC, f"--offload-arch={ARCH}", "-O1", "-g", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *SAN_HOST,
          "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, "lce_api.hip"),
          "-o", api_o])
    _run([clang, "-O1", "-g", "-std=c11", "-Wall", *SAN_C, "-D__HIP_PLATFORM_AMD__",
          "-I", os.path.join(ROOT, "include"), "-c", HOST_CHECKS_SRC, "-o", harness_o])
    tmp = HOST_CHECKS + ".tmp"
    _run([clang + "++", *SAN_C, "-o", tmp, harness_o, api_o, *objs,
          "-L", os.path.join(rocm, "lib"), "-lamdhip64",
          f"-Wl,-rpath,{os.path.join(rocm, 'lib')}"])
    os.replace(tmp, HOST_CHECKS)
    if verbose:
        print(f"built {HOST_CHECKS}")
    return HOST_CHECKS


if __name__ == "__main__":
    build(sanitize="--sanitize" in sys.argv[1:])
