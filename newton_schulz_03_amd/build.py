"""Builds libmuon_mi355x.so in-tree with hipcc for gfx950.

    python -m newton_schulz_03_amd.build [--verbose] [--save-temps DIR]

Every .hip file under csrc/ is compiled to an object (in parallel), then the
objects are linked into newton_schulz_03_amd/lib/libmuon_mi355x.so.  A second
library, libmuon_mi355x_tiletrace.so, links the same objects except the bf16
matrix-core source, compiled with -DMUON_TILE_TRACE: its kernels record a
per-workgroup timeline (`python bench.py --tile-timeline` reads it).  The
default library's kernels carry none of that code.
"""
from __future__ import annotations

import argparse
import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(PKG, "lib")
LIBNAME = "libmuon_mi355x.so"
TRACE_LIBNAME = "libmuon_mi355x_tiletrace.so"
TRACE_SOURCE = "gemm_bf16.hip"  # the one source with timeline hooks
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # packed fp32 instructions stay disabled: ordinary float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build the library")
    return path


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, save_temps: str | None, verbose: bool, trace: bool = False) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + (".trace.o" if trace else ".o"))
    cmd = [hipcc(), *HIPCC_FLAGS, *(["-DMUON_TILE_TRACE"] if trace else []), "-c", src, "-o", obj]
    if save_temps:
        os.makedirs(save_temps, exist_ok=True)
        cmd.insert(1, f"-save-temps={'obj'}")
        obj_dir = save_temps
        obj = os.path.join(obj_dir, os.path.basename(src) + (".trace.o" if trace else ".o"))
        cmd[-1] = obj
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, flush=True)
    return obj


def _link(objs, name: str, verbose: bool) -> str:
    out = os.path.join(LIBDIR, name)
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, out)
    return out


def build(verbose: bool = False, save_temps: str | None = None) -> str:
    """Compile every kernel source and link the shared library (and the
    timeline build beside it); returns the library's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    srcs = sources()
    jobs = [(s, False) for s in srcs] + [(os.path.join(CSRC, TRACE_SOURCE), True)]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(lambda j: _compile(j[0], save_temps, verbose, j[1]), jobs))
    plain, trace_obj = objs[:len(srcs)], objs[-1]
    out = _link(plain, LIBNAME, verbose)
    _link([trace_obj if os.path.basename(s) == TRACE_SOURCE else o for s, o in zip(srcs, plain)],
          TRACE_LIBNAME, verbose)
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--save-temps", default=None, help="keep hipcc intermediates (ISA) in DIR")
    args = ap.parse_args(argv)
    print(build(verbose=args.verbose, save_temps=args.save_temps))
    return 0


if __name__ == "__main__":
    sys.exit(main())
