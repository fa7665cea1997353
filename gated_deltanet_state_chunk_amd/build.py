"""Build libgdn.so (HIP, gfx950) in-tree.

    python -m gated_deltanet_state_chunk_amd.build [--resource-usage]

Each translation unit is compiled separately with hipcc and the objects are
linked into gated_deltanet_state_chunk_amd/libgdn.so.  Packed fp32 arithmetic
is disabled for the device code (-packed-fp32-ops); the host pass of hipcc
warns that it does not know that feature, which is harmless.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libgdn.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["gdn_chunk.hip", "gdn_decode.hip", "gdn_conv.hip", "gdn_pool.hip", "gdn_scratch.hip", "gdn_probe.hip", "gdn_api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
            "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-Wall", "-Wno-unused-result"]


def _compile(src: str, resource_usage: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), "-c", "-x", "hip", os.path.join(CSRC, src), "-o", obj] + common_flags()
    if resource_usage:
        cmd += ["-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(msgs))
    if resource_usage and msgs:
        print("\n".join(msgs), flush=True)
    return obj


def build(verbose: bool = False, resource_usage: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, resource_usage), SOURCES))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--resource-usage", action="store_true")
    a = ap.parse_args()
    print(build(verbose=True, resource_usage=a.resource_usage))
    sys.exit(0)
