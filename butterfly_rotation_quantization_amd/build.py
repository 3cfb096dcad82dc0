"""Build libbrq.so for gfx950 in-tree with hipcc.

    python -m butterfly_rotation_quantization_amd.build [-j N] [--verbose]

Every HIP source is compiled with packed-fp32 instruction selection disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); hipcc's host pass
warns that the feature is unknown to x86, which is harmless.
"""

from __future__ import annotations

import argparse
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libbrq.so")
DRYRUN_LIB = os.path.join(LIBDIR, "libbrq_dryrun.so")
DRYRUN_ASAN_LIB = os.path.join(LIBDIR, "libbrq_dryrun_asan.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def sources():
    """Sources of libbrq.so: every HIP kernel file and host file in csrc/."""
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def dryrun_sources():
    """Sources of libbrq_dryrun.so: the host layer with host memory in place of
    the device runtime and an index-walking checker in place of each launch."""
    host = [s for s in glob.glob(os.path.join(CSRC, "*.cpp"))
            if os.path.basename(s) != "runtime.cpp"]
    return sorted(host + glob.glob(os.path.join(CSRC, "dryrun", "*.cpp")))


# AddressSanitizer for the host code of the dry-run build (it holds no device
# code; the instrumentation is asked for the host side only).  The library
# leaves the sanitizer runtime unresolved: a process loads it first
# (LD_PRELOAD of asan_runtime()).
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
              "-Xarch_host", "-g"]


def asan_runtime() -> str:
    """Path of clang's AddressSanitizer runtime for x86-64 in the ROCm LLVM."""
    r = subprocess.run([os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm", "bin", "clang"),
                        "--print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        matches = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
        path = matches[-1] if matches else ""
    return path


def _compile(src: str, verbose: bool, objdir: str = OBJ, extra=()) -> str:
    obj = os.path.join(objdir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, *extra, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out, verbose):
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(jobs: int = 8, verbose: bool = False) -> str:
    """libbrq.so, its dry-run build and the dry-run build under AddressSanitizer."""
    dry_obj = os.path.join(OBJ, "dryrun")
    asan_obj = os.path.join(OBJ, "dryrun_asan")
    for d in (dry_obj, asan_obj, LIBDIR):
        os.makedirs(d, exist_ok=True)
    jobs_list = ([(s, OBJ, ()) for s in sources()] + [(s, dry_obj, ()) for s in dryrun_sources()] +
                 [(s, asan_obj, tuple(ASAN_FLAGS)) for s in dryrun_sources()])
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda sj: _compile(sj[0], verbose, sj[1], sj[2]), jobs_list))
    n, k = len(sources()), len(dryrun_sources())
    _link(objs[:n], LIB, verbose)
    _link(objs[n:n + k], DRYRUN_LIB, verbose)
    _link(objs[n + k:], DRYRUN_ASAN_LIB, verbose)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.j, a.verbose))


if __name__ == "__main__":
    sys.exit(main())
