"""Ahead-of-time build of libgsr.so (the C-ABI library) for gfx950.

Usage: python -m tiled_dense_gemm_scale_amd.build [--verbose]
"""
from __future__ import annotations

import argparse
import hashlib
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libgsr.so")
SOURCES = [os.path.join(CSRC, "gsr_api.hip")]
# The digest of the sources a build used is written beside the library, so a
# library older than its sources can be told apart from a current one.
DIGEST_SUFFIX = ".sources"


def depends() -> list:
    """Every file the library is compiled from: the kernel and launch sources
    and the public header."""
    return sorted(os.path.join(CSRC, n) for n in os.listdir(CSRC)) + [os.path.join(INCLUDE, "gsr.h")]


def source_digest() -> str:
    h = hashlib.sha256()
    for path in depends():
        with open(path, "rb") as f:
            h.update(os.path.relpath(path, ROOT).encode())
            h.update(f.read())
    return h.hexdigest()


def is_stale(output: str = LIBRARY) -> bool:
    """True when the library is missing, or was built from other sources than
    the current ones.  A library without a recorded digest (built elsewhere and
    copied in) is taken as it is."""
    if not os.path.exists(output):
        return True
    try:
        with open(output + DIGEST_SUFFIX) as f:
            return f.read().strip() != source_digest()
    except FileNotFoundError:
        return False


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise FileNotFoundError("hipcc not found (ROCm is required to build libgsr.so)")


def build(output: str = LIBRARY, verbose: bool = False, extra=()) -> str:
    cmd = [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           # no packed-fp32 VALU instructions anywhere in the device code
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", INCLUDE, "-I", CSRC, *extra, *SOURCES, "-o", output + ".tmp"]
    if verbose:
        cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err:
        print(err)
    digest = source_digest()
    os.replace(output + ".tmp", output)
    with open(output + DIGEST_SUFFIX, "w") as f:
        f.write(digest + "\n")
    return output


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--output", default=LIBRARY)
    args = ap.parse_args(argv)
    path = build(args.output, verbose=args.verbose)
    print(path)
    return 0


if __name__ == "__main__":
    sys.exit(main())
