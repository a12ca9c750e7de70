"""Build libmoe_ffn.so (gfx950 only) in the package directory with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe_ffn.so")
SOURCES = ["abi.hip", "layer.hip", "stream_read.hip", "mfma_rate.hip", "probes.hip", "attention.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")



def build(verbose: bool = False) -> str:
    """Compile every HIP source into one shared library; returns its path."""
    objs = []
    for src in SOURCES:
        obj = os.path.join(CSRC, "_build", src.replace(".hip", ".o"))
        os.makedirs(os.path.dirname(obj), exist_ok=True)
        # packed-fp32 instructions stay off: the compiler must not form v_pk_{add,mul,fma}_f32
        cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, stderr=subprocess.PIPE, text=True)
        if res.returncode != 0:
            print(res.stderr, flush=True)
            raise RuntimeError(f"hipcc failed on {src}")
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
