"""Build libska.so (HIP, gfx950) in-tree.

    python -m long_context_decode_ada_amd.build [--jobs N]

Compiles the kernel translation units and the host API with hipcc and links
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

UNITS = {
    "k_decode.hip": [],
    "k_codes.hip": ["-ffp-contract=off"],
    "k_rdr.hip": ["-ffp-contract=off"],
    "ska_api.cpp": ["-ffp-contract=off", "-fno-builtin"],
}


def _compile(src: str, extra: list) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"]
    cmd = ["hipcc", *lang, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    return obj


def build(jobs: int = 3, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda kv: _compile(*kv), UNITS.items()))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=3)
    args = ap.parse_args()
    build(args.jobs, verbose=True)
