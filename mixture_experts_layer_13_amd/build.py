"""Builds libmoe.so in-tree with hipcc for gfx950.

Usage: python mixture_experts_layer_13_amd/build.py [--host-sanitized]
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = ["csrc/api.hip", "csrc/route.hip", "csrc/ffn.hip", "csrc/ffn_stream.hip", "csrc/ffn_tiled.hip",
           "csrc/ffn_tiled256.hip", "csrc/ffn_tiled_int4.hip",
           "csrc/ffn_tiled_fp8.hip", "csrc/ffn_tiled_f8f8.hip"]
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


PROBE_SOURCE = "csrc/probe.hip"   # memory-system probes of the measurement harness (libmoe_probe.so)


def build(verbose: bool = False) -> str:
    """Compiles every source (in parallel) to objects under _build/ and links libmoe.so, and the
    probe library libmoe_probe.so beside it."""
    out = os.path.join(HERE, "libmoe.so")
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.basename(src).replace(".hip", ".o")) for src in SOURCES]
    cmds = [[HIPCC] + FLAGS + ["-c", os.path.join(HERE, src), "-o", obj] for src, obj in zip(SOURCES, objs)]
    probe_obj = os.path.join(objdir, "probe.o")
    cmds.append([HIPCC] + FLAGS + ["-c", os.path.join(HERE, PROBE_SOURCE), "-o", probe_obj])
    with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1)) as pool:
        msgs = list(pool.map(_run, cmds))
    tmp = out + ".tmp"
    msgs.append(_run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp]))
    probe_out = os.path.join(HERE, "libmoe_probe.so")
    msgs.append(_run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", probe_obj, "-o", probe_out + ".tmp"]))
    os.replace(probe_out + ".tmp", probe_out)
    if verbose and any(m.strip() for m in msgs):
        print("\n".join(m for m in msgs if m.strip()))
    os.replace(tmp, out)
    return out


HOST_SANITIZERS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                   "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]


def build_host_sanitized() -> str:
    """A second build of the library whose host code of the C ABI (csrc/api.hip: argument checks,
    planning, workspace carving, launch sequencing) carries AddressSanitizer and UBSan; the device
    code and the kernel launchers are the objects of the normal build (run build() first).  Load
    it with the ASan runtime preloaded (tests/test_host_sanitizers.py does)."""
    objdir = os.path.join(HERE, "_build")
    others = [os.path.join(objdir, os.path.basename(src).replace(".hip", ".o")) for src in SOURCES[1:]]
    missing = [o for o in others if not os.path.exists(o)]
    if missing:
        raise FileNotFoundError(f"build() first: {missing[0]} is missing")
    sandir = os.path.join(objdir, "hostsan")
    os.makedirs(sandir, exist_ok=True)
    api_obj = os.path.join(sandir, "api.o")
    flags = [f for f in FLAGS if f != "-O3"] + ["-O1", "-g"]
    _run([HIPCC] + flags + HOST_SANITIZERS + ["-c", os.path.join(HERE, SOURCES[0]), "-o", api_obj])
    out = os.path.join(sandir, "libmoe_hostsan.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + HOST_SANITIZERS[:4] + [api_obj] + others +
         ["-o", out])
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    if "--host-sanitized" in sys.argv:
        print(build_host_sanitized())
    sys.exit(0)
