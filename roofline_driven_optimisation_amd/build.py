"""Build libgemm.so (gfx950 only) from csrc/*.hip with hipcc.

Every source is compiled for ``--offload-arch=gfx950`` with packed-fp32 ops
disabled and linked into one shared library next to this file.  Object files
go to ``_build/`` beside the sources.
"""
from __future__ import annotations

import concurrent.futures as cf
import ctypes
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgemm.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-fvisibility=hidden",
    "-ffp-contract=fast", "-munsafe-fp-atomics",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + INCLUDE, "-I" + CSRC,
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str, extra, build_dir: str) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC] + CFLAGS + list(extra) + ["-c", src, "-o", obj]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s%s" % (src, proc.stdout, proc.stderr))
    return obj


def build(verbose: bool = False, extra=(), lib: str = LIB, build_dir: str = BUILD_DIR,
          check_load: bool = True) -> str:
    """Compile every kernel source and link libgemm.so; returns its path.
    ``extra`` flags go to every compile and the link; ``lib`` and
    ``build_dir`` place a variant build elsewhere (a host-sanitizer build,
    which loads only with its runtime preloaded: ``check_load=False``)."""
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, build_dir), srcs))
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC"] + list(extra) + ["-o", tmp] + objs
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError("link failed:\n%s%s" % (proc.stdout, proc.stderr))
    # a kernel whose host stub was not emitted only shows up at load time
    if check_load:
        try:
            ctypes.CDLL(tmp)
        except OSError as exc:
            os.unlink(tmp)
            raise RuntimeError("built library does not load: %s" % exc)
    os.replace(tmp, lib)
    if verbose:
        print("built", lib)
    return lib


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
