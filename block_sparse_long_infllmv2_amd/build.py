"""Builds libinfllmv2.so (gfx950) in-tree with hipcc.

    python -m block_sparse_long_infllmv2_amd.build [--jobs N]

Every HIP source under csrc/ is compiled to an object in parallel, then linked
into block_sparse_long_infllmv2_amd/libinfllmv2.so.  Packed float32 vector
instructions are disabled for all device code.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libinfllmv2.so")
OBJDIR = os.path.join(ROOT, "_build", "obj")
# the same sources with -DINFLLMV2_DEBUG: every attention call first checks
# the kept-block rows and tree masks it consumes (infllmv2_debug_check)
DEBUG_LIB = os.path.join(HERE, "libinfllmv2_debug.so")
DEBUG_OBJDIR = os.path.join(ROOT, "_build", "obj_debug")

ARCH = "gfx950"
CXXFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str, hipcc: str, debug: bool = False) -> str:
    obj = os.path.join(DEBUG_OBJDIR if debug else OBJDIR, os.path.basename(src) + ".o")
    cmd = [hipcc, *CXXFLAGS, *(["-DINFLLMV2_DEBUG"] if debug else []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(ln for ln in (r.stderr or "").splitlines()
                     if "packed-fp32-ops" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
    if errs.strip():
        sys.stderr.write(errs + "\n")
    return obj


PROBES = os.path.join(HERE, "probes")


def build_probes(hipcc: str) -> list:
    """Stand-alone measurement programs (probes/*.hip -> probes/<name>): not
    part of the library, built so that their results can be reproduced."""
    out = []
    for src in sorted(glob.glob(os.path.join(PROBES, "*.hip"))):
        exe = src[:-len(".hip")]
        cmd = [hipcc, "-O3", "-std=c++17", f"--offload-arch={ARCH}",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-o", exe, src]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        out.append(exe)
    return out


def _check_loads(path: str) -> None:
    """Resolve every symbol of the built library now, in a child process (no
    GPU is touched): a kernel whose host-side launch stub was not emitted
    links, but leaves an undefined symbol that only loading reveals."""
    code = "import ctypes, os, sys; ctypes.CDLL(sys.argv[1], mode=os.RTLD_NOW)"
    r = subprocess.run([sys.executable, "-c", code, path], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{path} does not load:\n{r.stderr.strip().splitlines()[-1]}")


def _link(objs: list, lib: str, hipcc: str) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    _check_loads(tmp)
    os.replace(tmp, lib)


def build(jobs: int = 8, verbose: bool = True, debug: bool = True) -> str:
    """Compile every csrc/*.hip and link libinfllmv2.so, the debug build
    libinfllmv2_debug.so (unless debug=False) and the probes; returns the
    library's path."""
    hipcc = _hipcc()
    os.makedirs(OBJDIR, exist_ok=True)
    os.makedirs(DEBUG_OBJDIR, exist_ok=True)
    srcs = sources()
    jobs_list = [(s, False) for s in srcs] + ([(s, True) for s in srcs] if debug else [])
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda sd: _compile(sd[0], hipcc, sd[1]), jobs_list))
    _link(objs[:len(srcs)], LIB, hipcc)
    if debug:
        _link(objs[len(srcs):], DEBUG_LIB, hipcc)
    probes = build_probes(hipcc)
    if verbose:
        print(f"built {LIB}{' and ' + DEBUG_LIB if debug else ''} from {len(srcs)} sources, "
              f"{len(probes)} probe(s)")
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--no-debug", action="store_true", help="skip the debug build")
    args = ap.parse_args()
    build(args.jobs, debug=not args.no_debug)
