"""Compile the HIP sources in ``csrc/`` into ``libkvc.so`` next to this file,
and the streaming-read probe in ``probe/`` into ``probe/libkvc_probe.so``.

gfx950 only.  Every source is built with the packed-fp32 target feature
switched off (the compiler would otherwise fuse pairs of fp32 operations into
packed instructions on its own).  Objects go to ``_build/`` at the repository
root; the shared object lands in the package directory so that the binding
finds it without any installation step.

    python -m kv_cached_decode_kvc_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build", "kvc")
LIB = os.path.join(PKG, "libkvc.so")
PROBE_DIR = os.path.join(PKG, "probe")
PROBE_LIB = os.path.join(PROBE_DIR, "libkvc_probe.so")
ARCH = "gfx950"

CFLAGS = ["--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I" + os.path.join(ROOT, "include")]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def sources(d: str = CSRC):
    return sorted(os.path.join(d, f) for f in os.listdir(d) if f.endswith(".hip"))


def _compile(src: str, include: str = "") -> str:
    obj = os.path.join(OBJ, os.path.basename(src)[:-4] + ".o")
    cmd = [hipcc(), *CFLAGS, *(["-I" + include] if include else []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s" % (src, out))
    if out.strip():
        print(out, file=sys.stderr)
    return obj


def _link(objs, lib: str):
    tmp = lib + ".tmp%d" % os.getpid()
    subprocess.check_call([hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs,
                           "-o", tmp])
    os.replace(tmp, lib)


def build(verbose: bool = True) -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    probe_srcs = sources(PROBE_DIR)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs) + len(probe_srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
        probe_objs = list(ex.map(lambda f: _compile(f, PROBE_DIR), probe_srcs))
    _link(objs, LIB)
    _link(probe_objs, PROBE_LIB)
    if verbose:
        print("built", LIB, "and", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    build()
