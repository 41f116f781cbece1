"""Build the packkv HIP library for gfx950, in-tree.

``python -m decode_gemv_amd.build`` (or ``build()``) compiles every HIP source
under ``csrc/`` with hipcc and links ``decode_gemv_amd/libpackkv.so``.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")
LIB = os.path.join(PKG, "libpackkv.so")
ARCH = "gfx950"
SOURCES = ["encode.hip", "gemv.hip", "api.hip"]

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC",
    # packed fp32 instructions stay off on this hardware
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", f"-I{INCLUDE}",
]
# the encoder must round exactly like the fp64 oracle: no contraction, no fast math
PER_SOURCE = {"encode.hip": ["-ffp-contract=off", "-fno-fast-math"]}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "is not a recognized feature for this target" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{errs}")
    if verbose and errs.strip():
        print(errs, file=sys.stderr)


# AddressSanitizer on the host code only (argument checks, sizes, launches);
# the device code is built as usual
HOST_ASAN = "-Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer".split()


def build(verbose: bool = False, out: str = LIB, host_asan: bool = False) -> str:
    """Compile all sources and link the shared library; returns its path.
    host_asan: instrument the host code with AddressSanitizer (load the
    library with the sanitizer runtime preloaded)."""
    hipcc = _hipcc()
    extra = HOST_ASAN if host_asan else []
    with tempfile.TemporaryDirectory(prefix="packkv_build_") as tmp:
        objs = []
        cmds = []
        for src in SOURCES:
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            objs.append(obj)
            cmds.append([hipcc, *COMMON, *extra, *PER_SOURCE.get(src, []), "-c",
                         os.path.join(CSRC, src), "-o", obj])
        with concurrent.futures.ThreadPoolExecutor(len(cmds)) as ex:
            list(ex.map(lambda c: _run(c, verbose), cmds))
        out_tmp = out + ".tmp"
        _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra[:2], *objs, "-o", out_tmp], verbose)
        os.replace(out_tmp, out)
    return out


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser(description="build libpackkv.so for gfx950")
    ap.add_argument("--out", default=LIB, help="library path (default: the in-tree one)")
    ap.add_argument("--host-asan", action="store_true", help="AddressSanitizer on the host code")
    args = ap.parse_args()
    print(build(verbose=True, out=args.out, host_asan=args.host_asan))
