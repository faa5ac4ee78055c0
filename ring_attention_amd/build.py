"""Build librattn.so (gfx950) in-tree with hipcc.

    python -m ring_attention_amd.build

Each .hip translation unit is compiled separately (in parallel) and then
linked into ring_attention_amd/librattn.so.  Every device compile disables
packed-FP32 instruction selection, so no v_pk_{add,mul,fma}_f32 is emitted.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ = os.path.join(ROOT, "_build", "rattn")
LIB = os.path.join(PKG, "librattn.so")
ARCH = os.environ.get("RATTN_OFFLOAD_ARCH", "gfx950")

SOURCES = ["rattn_abi.hip", "fwd_generic.hip", "fwd_mfma.hip", "fwd_mfma128.hip", "fwd_short.hip", "merge.hip",
           "bwd_generic.hip", "bwd_mfma.hip"]

COMMON = ["-std=c++17", "-O3", "-fPIC", "-fvisibility=hidden", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-result", "-I", INCLUDE, "-I", CSRC]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build librattn")
    return exe


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    err = "\n".join(line for line in r.stderr.splitlines()
                    if "packed-fp32-ops" not in line and line.strip())
    if verbose and err:
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    jobs = min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8") or 8))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


# ---- sanitizer builds of the host code (CPU-only checks) --------------------
#
# The library's host code (argument checks, schedule building, size
# arithmetic) compiled with AddressSanitizer and UndefinedBehaviorSanitizer,
# linked with the regular device objects, and two drivers that exercise it and
# the CPU oracle without a GPU (tests/sanitize/, run by tests/test_sanitize.py).
# The sanitizers apply to host code only: every -fsanitize on a hipcc line
# follows -Xarch_host.

SAN_DIR = os.path.join(ROOT, "_build", "sanitize")
SAN_LIB = os.path.join(SAN_DIR, "librattn_san.so")
SAN_ABI_DRIVER = os.path.join(SAN_DIR, "abi_driver")
SAN_ORACLE_DRIVER = os.path.join(SAN_DIR, "oracle_driver")
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _stale(target: str, sources: list) -> bool:
    if not os.path.exists(target):
        return True
    t = os.path.getmtime(target)
    return any(os.path.getmtime(x) > t for x in sources)


def _run(cmd: list, verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitizer build failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")


def build_sanitize_checks(verbose: bool = False) -> tuple:
    """Build (if out of date) the sanitized library copy and both drivers;
    returns the paths of the ABI driver and the oracle driver."""
    os.makedirs(SAN_DIR, exist_ok=True)
    tests = os.path.join(ROOT, "tests", "sanitize")
    csrc = [os.path.join(CSRC, f) for f in os.listdir(CSRC)]
    headers = [os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE)]
    abi_driver_src = os.path.join(tests, "abi_driver.c")
    if _stale(SAN_LIB, csrc + headers):
        objs = [os.path.join(OBJ, os.path.splitext(x)[0] + ".o") for x in SOURCES
                if x != "rattn_abi.hip"]
        if any(_stale(o, csrc + headers) for o in objs):
            build(verbose)
        abi_obj = os.path.join(SAN_DIR, "rattn_abi_san.o")
        _run([hipcc(), *COMMON, *SANITIZE_HOST, "-c", os.path.join(CSRC, "rattn_abi.hip"),
              "-o", abi_obj], verbose)
        _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", abi_obj, *objs,
              "-o", SAN_LIB], verbose)
    if _stale(SAN_ABI_DRIVER, [SAN_LIB, abi_driver_src]):
        clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin",
                             "clang")
        if not os.path.exists(clang):
            clang = "/opt/rocm/llvm/bin/clang"
        _run([clang, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
              "-fno-omit-frame-pointer", "-I", INCLUDE, abi_driver_src, SAN_LIB,
              f"-Wl,-rpath,{SAN_DIR}", "-o", SAN_ABI_DRIVER], verbose)
    oracle_c = os.path.join(ROOT, "oracle", "oracle.c")
    oracle_driver_src = os.path.join(tests, "oracle_driver.c")
    if _stale(SAN_ORACLE_DRIVER, [oracle_c, oracle_driver_src]):
        _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address,undefined",
              "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", oracle_driver_src, oracle_c,
              "-lm", "-o", SAN_ORACLE_DRIVER], verbose)
    return SAN_ABI_DRIVER, SAN_ORACLE_DRIVER


if __name__ == "__main__":
    print(build(verbose=True))
