"""Build libska.so (HIP, gfx950) in-tree.

    python -m long_context_decode_ada_amd.build [--jobs N]

Compiles the kernel translation units (the decode kernels once per head
dimension and group size) and the host API with hipcc and links
them into long_context_decode_ada_amd/libska.so.  The encode/query-code unit
and the host API are built with -ffp-contract=off (their binary64 decisions
must be rounded exactly as written); the decode unit may contract.
"""
from __future__ import annotations

import argparse
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libska.so")
ARCH = os.environ.get("SKA_OFFLOAD_ARCH", "gfx950")

COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-I" + os.path.join(ROOT, "include"),
          # packed fp32 VALU ops are kept out of the generated code
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument"]

# (object name, source, extra flags).  The decode kernel families (head
# dimension x group size x query precision) are one source built once per
# family, so that they compile in parallel.
UNITS = [(f"k_decode_{d}_{g}_{q}", "k_decode_inst.hip", [f"-DSKA_INST_D={d}", f"-DSKA_INST_G={g}", f"-DSKA_INST_QF={q}"])
         for d in (128, 64) for g in (4, 2, 1) for q in (0, 1)] + [
    ("k_decode", "k_decode.hip", []),
    ("k_codes", "k_codes.hip", ["-ffp-contract=off"]),
    ("k_rdr", "k_rdr.hip", ["-ffp-contract=off"]),
    ("ska_api", "ska_api.cpp", ["-ffp-contract=off", "-fno-builtin"]),
]


def _compile(name: str, src: str, extra: list) -> str:
    obj = os.path.join(BUILD, name + ".o")
    lang = ["-x", "hip"]
    cmd = ["hipcc", *lang, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    return obj


def build(jobs: int = 0, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    if jobs <= 0:
        jobs = min(len(UNITS), os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda u: _compile(*u), UNITS))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


def build_abi_sanitized(verbose: bool = False) -> str:
    """A program that drives the C ABI's host checks (tests/abi_sanitize_main.c)
    linked with the host API built with AddressSanitizer and
    UndefinedBehaviorSanitizer on its host code (device code unchanged) and
    the kernel objects of build().  Returns the program's path."""
    if not all(os.path.exists(os.path.join(BUILD, n + ".o")) for n, _, _ in UNITS):
        build()
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    obj = os.path.join(BUILD, "ska_api_sanitized.o")
    flags = [f for n, src, f in UNITS if src == "ska_api.cpp"][0]
    cmd = ["hipcc", "-x", "hip", *COMMON, *flags, *san, "-O1", "-g", "-c", os.path.join(CSRC, "ska_api.cpp"),
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s" % (" ".join(cmd), r.stderr))
    exe = os.path.join(BUILD, "abi_sanitize")
    objs = [os.path.join(BUILD, n + ".o") for n, src, _ in UNITS if src != "ska_api.cpp"]
    cmd = ["hipcc", f"--offload-arch={ARCH}", *san, "-g", "-x", "c", os.path.join(ROOT, "tests", "abi_sanitize_main.c"),
           "-x", "none", obj, *objs, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s" % (" ".join(cmd), r.stderr))
    if verbose:
        print("built", exe)
    return exe


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=0, help="parallel compiles (0: one per CPU, at most one per unit)")
    args = ap.parse_args()
    build(args.jobs, verbose=True)
