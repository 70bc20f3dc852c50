"""Build libtaq.so (HIP for gfx950) in-tree.

    python -m tiled_attention_quantized_amd.build

Each source is compiled separately (in parallel) and linked into
``tiled_attention_quantized_amd/libtaq.so``.  Objects go to ``_build/``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libtaq.so")
SOURCES = ["api.hip", "kv_quant.hip", "attn_decode.hip", "attn_prefill.hip", "tile_mask.hip",
           "head_precision.hip"]
ARCH = "gfx950"

# packed-fp32-ops is switched off for every device compile: the VOP3P packed
# fp32 forms are left to nobody, and scalar fp32 code is what the kernels need.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for p in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if p and os.path.exists(p):
            return p
    raise RuntimeError("hipcc not found")


def _compile(src: str, extra, build_dir: str) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
           "-Wall", "-Wno-unused-function", *DEVICE_FLAGS, *extra,
           "-I", os.path.join(PKG, "..", "include"),
           "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile of {src} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, extra=(), lib_path: str = LIB, build_dir: str = BUILD) -> str:
    """Compile every source and link ``lib_path``.  ``extra`` are additional
    hipcc flags (for example -D overrides of the kernels' tuning knobs)."""
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra), build_dir), SOURCES))
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib_path)
    if verbose:
        print(f"built {lib_path}")
    return lib_path


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
