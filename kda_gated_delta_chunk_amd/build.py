"""Build libkda.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc.

Every translation unit under csrc/ is compiled for gfx950 in parallel and
linked into one shared library next to this file. Packed-fp32 instruction
selection is switched off for all device code.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
CSRC = PKG / "csrc"
LIB = PKG / "libkda.so"
SOURCES = ["kda_prefill.hip", "kda_decode.hip", "kda_backward.hip", "kda_api.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops' is not a recognized" not in l)
    if r.returncode != 0:
        raise RuntimeError("command failed: %s\n%s" % (" ".join(cmd), out))
    return out


def build(verbose: bool = False) -> Path:
    """Compile all sources and link libkda.so; returns its path."""
    objdir = PKG / "_build"
    objdir.mkdir(exist_ok=True)
    objs = [objdir / (s.rsplit(".", 1)[0] + ".o") for s in SOURCES]
    cmds = [[HIPCC, *FLAGS, "-c", str(CSRC / s), "-o", str(o)] for s, o in zip(SOURCES, objs)]
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB.with_suffix(".so.tmp%d" % os.getpid())
    _run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", str(tmp), *map(str, objs)])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
