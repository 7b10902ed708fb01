"""Build libbdd.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m block_diffusion_decode_amd.build [--jobs N] [--verbose]

Each .hip source is compiled to an object under _build/ and linked into
block_diffusion_decode_amd/libbdd.so.  hipcc cross-compiles for gfx950 without
a GPU.  Packed fp32 VALU instructions are disabled for device code.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libbdd.so")
SOURCES = ["route.hip", "experts.hip", "lmhead.hip", "api.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libbdd.so)")


def compile_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function", "-Wno-pass-failed",
        "-I", os.path.join(ROOT, "include"),
    ]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the device feature flag: drop that note
    out = "\n".join(l for l in p.stdout.splitlines() if "is not a recognized feature" not in l)
    return p.returncode, out


def build(jobs: int = 4, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([cc, *compile_flags(), "-c", os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        results = list(ex.map(lambda c: _run(c, verbose), cmds))
    for (rc, out), cmd in zip(results, cmds):
        if out.strip():
            print(out, file=sys.stderr)
        if rc != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}")
    tmp = LIB + ".tmp"
    rc, out = _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    if out.strip():
        print(out, file=sys.stderr)
    if rc != 0:
        raise RuntimeError("link failed")
    os.replace(tmp, LIB)
    return LIB


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("--verbose", action="store_true")
    a = ap.parse_args()
    print(build(a.jobs, a.verbose))


if __name__ == "__main__":
    main()
