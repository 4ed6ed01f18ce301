"""Build the gfx950 shared library libagent_attn.so in-tree with hipcc.

    python -m efficient_attention_vision_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libagent_attn.so")
SOURCES = (["agent_attn.hip"] + [f"mfma_dc{dc}_{t}.hip" for dc in (1, 2, 4)
                                for t in ("bf16", "f16")]
           + [f"bwd_mfma_{t}.hip" for t in ("bf16", "f16")] + ["proj.hip"])
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMPILE_FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
    # the packed-fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _filter(out: str) -> str:
    # hipcc's host pass does not know the packed-fp32 feature and says so
    return "\n".join(l for l in out.splitlines()
                     if "packed-fp32-ops' is not a recognized feature" not in l)


def build(verbose: bool = False, extra_flags=(), output: str = LIB) -> str:
    """Compile every source to an object in parallel, then link the library."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, *COMPILE_FLAGS, *extra_flags, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                 stderr=subprocess.STDOUT, text=True)))
    objs = []
    for src, obj, pr in procs:
        out, _ = pr.communicate()
        out = _filter(out)
        if pr.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src} ({pr.returncode}):\n{out}")
        if verbose and out.strip():
            print(out)
        objs.append(obj)
    tmp = output + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed ({r.returncode}):\n{_filter(r.stdout)}")
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
