"""Build libfcm.so (the C ABI + gfx950 kernels) in-tree with hipcc.

    python -m depthwise_pointwise_convolution_amd.build [--jobs N]

Each translation unit is compiled to an object under ``_build/`` in parallel and
the objects are linked into ``depthwise_pointwise_convolution_amd/libfcm.so``.
Device code is built for gfx950 only, with packed fp32 arithmetic disabled.  Every
kernel source is also compiled to gfx950 assembly, which isa_check.py inspects; the
library is refused if a store of more than 64 bits is directly followed by a write of
its data registers (see isa_check.py).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfcm.so")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")

SOURCES = [
    ("kernels/dwpw.hip", True),
    ("kernels/dwpw_mm.hip", True),
    ("kernels/dwpw_mmw.hip", True),
    ("kernels/dwpw_ws.hip", True),
    ("kernels/dwpw_wsl.hip", True),
    ("kernels/b2b_mm.hip", True),
    ("kernels/pwdw_mm.hip", True),
    ("kernels/pwdwpw_mm.hip", True),
    ("kernels/dwpw_i8.hip", True),
    ("kernels/pwpw_mm.hip", True),
    ("kernels/dwpw_gen.hip", True),
    ("kernels/lbl.hip", True),
    ("kernels/b2b.hip", True),
    ("api.cpp", True),
    ("plan.cpp", False),
]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the gfx950 library cannot be built")


def _flags(device: bool) -> list:
    f = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
         "-I" + INCLUDE, "-I" + CSRC]
    if device:
        f = ["-x", "hip", "--offload-arch=gfx950", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", "-munsafe-fp-atomics"] + f
    return f


def _compile(src: str, device: bool, verbose: bool) -> str:
    os.makedirs(BUILD, exist_ok=True)
    obj = os.path.join(BUILD, src.replace("/", "_") + ".o")
    cmd = [_hipcc()] + _flags(device) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{out}")
    if out.strip() and verbose:
        print(out)
    return obj


def _check_isa(src: str) -> list:
    """gfx950 assembly of one kernel source, checked by isa_check."""
    try:
        from .isa_check import store_data_overwrites
    except ImportError:  # loaded by path rather than as part of the package
        sys.path.insert(0, PKG)
        from isa_check import store_data_overwrites
    os.makedirs(BUILD, exist_ok=True)
    asm = os.path.join(BUILD, src.replace("/", "_") + ".s")
    cmd = [_hipcc()] + _flags(True) + ["--cuda-device-only", "-S", os.path.join(CSRC, src),
                                        "-o", asm]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} to assembly failed:\n{r.stderr}")
    with open(asm) as f:
        return [(src,) + hit for hit in store_data_overwrites(f.read())]


def build(jobs: int = 0, verbose: bool = False) -> str:
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4)
    kernels = [s for s, dev in SOURCES if s.startswith("kernels/")]
    with cf.ThreadPoolExecutor(jobs) as ex:
        checks = [ex.submit(_check_isa, k) for k in kernels]
        objs = list(ex.map(lambda s: _compile(s[0], s[1], verbose), SOURCES))
        hits = [h for c in checks for h in c.result()]
    if hits:
        src, fn, reader, writer = hits[0]
        raise RuntimeError(f"{len(hits)} store(s) of more than 64 bits would have their data "
                           f"registers rewritten by the next instruction, e.g. in {src} {fn}:"
                           f"\n  {reader}\n  {writer}")
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("linking libfcm.so failed:\n" + r.stdout + r.stderr)
    # a kernel template whose host launch stub was never emitted leaves an undefined
    # symbol that only fails when the library is loaded: refuse such a link here
    nm = shutil.which("nm") or "/opt/rocm/llvm/bin/llvm-nm"
    r = subprocess.run([nm, "-D", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [l.split()[-1] for l in r.stdout.splitlines() if "fcm" in l]
    if r.returncode != 0 or missing:
        os.remove(tmp)
        raise RuntimeError("libfcm.so would have undefined symbols: " + " ".join(missing[:8]))
    os.replace(tmp, LIB)
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=0)
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args(argv)
    print(build(args.jobs, args.verbose))
    return 0


if __name__ == "__main__":
    sys.exit(main())
