"""Build libforge.so (the HIP kernels + C ABI) in place for gfx950 with hipcc."""
from __future__ import annotations

import hashlib
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libforge.so")

# -ffp-contract=off: every fused multiply-add is written out explicitly, so the fused and
# the unfused kernels round identically.  The packed-fp32 target feature is switched off.
DEVICE_FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-ffp-contract=off",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# The fused kernels of each path and moment / input format are instantiated in their own
# translation unit, so the sources compile in parallel.
SOURCES = ["forge_fused2_q8.hip", "forge_fused2_q8d.hip", "forge_fused1_f32.hip", "forge_fused1_bf16.hip",
           "forge_fused1_fp8.hip", "forge_fused8_q8.hip", "forge_fused8_q8d.hip", "forge_fused2_f32.hip",
           "forge_fused8_f32.hip", "forge_backward.hip", "forge_kernels.hip", "forge_measure.hip", "forge_host.cpp"]


def source_hash(root: str = ROOT) -> str:
    """Hash of every library source (csrc/ and include/ under `root`); the build embeds it as
    forge_build_id()."""
    h = hashlib.sha256()
    for d in (os.path.join(root, "optimizer_step_weight_amd", "csrc"), os.path.join(root, "include")):
        for f in sorted(os.listdir(d)):
            if f.endswith((".h", ".hip", ".cpp")):
                with open(os.path.join(d, f), "rb") as fh:
                    h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str, verbose: bool, build_id: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *DEVICE_FLAGS, f'-DFORGE_BUILD_ID="{build_id}"', "-I" + INCLUDE, "-I" + CSRC, "-c",
           os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    build_id = source_hash()
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4, 16)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_id), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
