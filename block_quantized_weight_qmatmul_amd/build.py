"""Build the HIP library (libqmv.so) in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "qmv.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libqmv.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
         # keep packed fp32 VALU ops out of the generated code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(out: str = LIB, extra: list[str] | None = None, quiet: bool = True) -> str:
    """Compile csrc/qmv.hip into ``out`` (atomically replaced)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, *(extra or []), "-I", INCLUDE, SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stdout + r.stderr)
    if not quiet:
        print(" ".join(cmd))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(quiet=False))
