"""Builds libmoe.so in-tree with hipcc for gfx950.

Usage: python mixture_experts_layer_13_amd/build.py
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = ["csrc/api.hip", "csrc/route.hip", "csrc/ffn.hip", "csrc/ffn_stream.hip", "csrc/ffn_tiled.hip",
           "csrc/ffn_tiled_int4.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         # packed fp32 VALU forms stay off for every HIP file of this library
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + msgs)
    return msgs


def build(verbose: bool = False) -> str:
    """Compiles every source (in parallel) to objects under _build/ and links libmoe.so."""
    out = os.path.join(HERE, "libmoe.so")
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.basename(src).replace(".hip", ".o")) for src in SOURCES]
    cmds = [[HIPCC] + FLAGS + ["-c", os.path.join(HERE, src), "-o", obj] for src, obj in zip(SOURCES, objs)]
    with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1)) as pool:
        msgs = list(pool.map(_run, cmds))
    tmp = out + ".tmp"
    msgs.append(_run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp]))
    if verbose and any(m.strip() for m in msgs):
        print("\n".join(m for m in msgs if m.strip()))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
