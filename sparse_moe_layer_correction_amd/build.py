"""Compile the HIP sources into the in-tree shared library (gfx950 only).

    python -m sparse_moe_layer_correction_amd.build

Each source is compiled in its own hipcc process, then linked into
``sparse_moe_layer_correction_amd/libmoe_mi355x.so``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libmoe_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["router.hip", "permute.hip", "gemm.hip", "skinny.hip", "combine.hip", "mx.hip", "norm.hip", "moe_api.hip"]

# -packed-fp32-ops: keep hipcc from forming packed fp32 instructions
COMMON_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, extra_flags=None) -> str:
    out_dir = os.path.join(ROOT, "_build")
    os.makedirs(out_dir, exist_ok=True)
    cc = hipcc()
    flags = COMMON_FLAGS + ["-I", INCLUDE, "-I", CSRC] + list(extra_flags or [])
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(out_dir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [cc] + flags + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        msg = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append((src, msg))
        elif verbose and msg.strip():
            print(msg)
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n".join(f"--- {s}\n{m}" for s, m in failed))
    tmp = LIB_PATH + ".tmp"
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
