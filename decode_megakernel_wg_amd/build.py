"""Build the HIP library libmk.so in-tree for gfx950 (hipcc; no JIT, no torch extension)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmk.so")
SOURCES = ["mk_kernel.hip", "mk_static.hip", "mk_host.cpp", "mk_plan.cpp"]

HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC", "-shared",
               # packed fp32 instructions are kept out of the generated code on purpose
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wno-unused-result"]


def build(verbose: bool = False, extra=()) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    cmd = ["hipcc", *HIPCC_FLAGS, *extra, *srcs, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs)
    os.replace(LIB + ".tmp", LIB)
    return LIB


PROBE_SRC = os.path.join(HERE, "hop_probe.hip")
PROBE = os.path.join(HERE, "hop_probe")


def build_probe(verbose: bool = False) -> str:
    """The measurement program hop_probe.hip (synchronisation and streaming costs; not part of the decode path)."""
    flags = [f for f in HIPCC_FLAGS if f not in ("-fPIC", "-shared")]
    cmd = ["hipcc", *flags, PROBE_SRC, "-o", PROBE + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        errs = "\n".join(l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l)
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{errs}")
    os.replace(PROBE + ".tmp", PROBE)
    return PROBE


if __name__ == "__main__":
    build(verbose=True)
    build_probe(verbose=True)
