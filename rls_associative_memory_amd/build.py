"""Build the HIP C-ABI library ``librls_vla.so`` in-tree for gfx950.

    python -m rls_associative_memory_amd.build [--verbose]

Every source is compiled with hipcc for --offload-arch=gfx950 and linked into
``rls_associative_memory_amd/lib/librls_vla.so``.  Packed-FP32 VALU instruction selection
is switched off for device code (``-target-feature -packed-fp32-ops``).
"""

from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(PKG, "lib")
BUILDDIR = os.path.join(PKG, "_build")
LIBNAME = "librls_vla.so"

SOURCES = ["vla_api.cpp", "vla_profile.cpp", "vla_seq.hip", "vla_chunk.hip", "vla_decode.hip", "la_chunk.hip", "vla_backward.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def common_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC,
        "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
    ]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n"
                           f"{res.stdout}\n{res.stderr}")
    err = "\n".join(line for line in res.stderr.splitlines()
                    if "packed-fp32-ops" not in line and line.strip())
    if verbose and err:
        print(err, file=sys.stderr)
    return res


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source and link the shared library; returns its path."""
    cc = hipcc()
    os.makedirs(BUILDDIR, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILDDIR, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"]
        cmds.append([cc, *common_flags(), *lang, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    out = os.path.join(LIBDIR, LIBNAME)
    tmp = out + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, out)
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--jobs", type=int, default=4)
    args = ap.parse_args()
    print(build(verbose=args.verbose, jobs=args.jobs))


if __name__ == "__main__":
    main()
