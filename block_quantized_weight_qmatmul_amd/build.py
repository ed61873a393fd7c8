"""Build the HIP library (libqmv.so) in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", f) for f in ("qmv.hip", "qmv_mq.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libqmv.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         # keep packed fp32 VALU ops out of the generated code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(out: str = LIB, extra: list[str] | None = None, quiet: bool = True) -> str:
    """Compile csrc/*.hip into ``out`` (atomically replaced): each source to an
    object file in parallel, then one link."""
    objs, procs = [], []
    for src in SRCS:
        obj = os.path.join(PKG, "csrc", os.path.basename(src) + ".o.tmp%d" % os.getpid())
        cmd = [HIPCC, *FLAGS, "-c", *(extra or []), "-I", INCLUDE, src, "-o", obj]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        objs.append(obj)
    try:
        for cmd, p in procs:
            o, e = p.communicate()
            if p.returncode != 0:
                raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + o + e)
            if not quiet:
                print(" ".join(cmd))
        tmp = out + ".tmp%d" % os.getpid()
        cmd = [HIPCC, *FLAGS, "-shared", *objs, "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc link failed:\n" + r.stdout + r.stderr)
        if not quiet:
            print(" ".join(cmd))
        os.replace(tmp, out)
    finally:
        for obj in objs:
            if os.path.exists(obj):
                os.remove(obj)
    return out


if __name__ == "__main__":
    print(build(quiet=False))
