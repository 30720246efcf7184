"""Build libsaga.so (HIP, gfx950) in-tree with hipcc.

Every .hip file under csrc/ is compiled to an object for gfx950 and linked
into sparse_asymmetric_gqa_amd/libsaga.so. Packed fp32 VALU instructions are
disabled for device code (-packed-fp32-ops).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsaga.so")
OBJDIR = os.path.join(PKG, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str, objdir: str = OBJDIR, extra=()) -> str:
    obj = os.path.join(objdir, os.path.basename(src).replace(".hip", ".o"))
    cmd = [HIPCC, *CFLAGS, "-I", os.path.dirname(src), *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in r.stderr.splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
    if errs:
        sys.stderr.write(errs + "\n")
    return obj


def build(verbose: bool = False, out: str = LIB, objdir: str = OBJDIR, extra=(),
          csrc: str = CSRC) -> str:
    """Compile all HIP sources and link libsaga.so; returns the library path.

    `extra` adds compiler flags (e.g. -D overrides of tile constants) and
    `out` / `objdir` / `csrc` redirect the products and sources, for building
    experimental variants next to the default library.
    """
    os.makedirs(objdir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(csrc, "*.hip")))
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s_: _compile(s_, objdir, tuple(extra)), srcs))
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True)
