"""Build libmoe_int4.so (hipcc, gfx950) in-tree.

Usage: python -m quantized_moe_router_amd.build
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libmoe_int4.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 instructions in any generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def build(verbose: bool = False) -> str:
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc")]
    objs = []
    procs = []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmd = [HIPCC, *FLAGS, *inc, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd, stderr=subprocess.PIPE, text=True), src))
        objs.append(obj)
    failed = False
    for p, src in procs:
        _, err = p.communicate()
        msgs = [l for l in err.splitlines() if "packed-fp32-ops" not in l]
        if p.returncode != 0:
            failed = True
            sys.stderr.write(f"--- {src}\n" + "\n".join(msgs) + "\n")
        elif verbose and msgs:
            sys.stderr.write("\n".join(msgs) + "\n")
    if failed:
        raise RuntimeError("hipcc failed")
    tmp = LIB + ".tmp"
    # --no-undefined: a kernel whose host stub was not emitted fails here, not at load time
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,--no-undefined", *objs,
                           "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
