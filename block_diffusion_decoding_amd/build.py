"""Build ``libbd.so`` (the C-ABI library) in-tree with hipcc for gfx950.

``python -m block_diffusion_decoding_amd.build`` compiles every source under
``csrc/`` to an object in ``_build/`` (in parallel) and links
``block_diffusion_decoding_amd/libbd.so``.  hipcc cross-compiles, so no GPU is
needed.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libbd.so")
INCLUDE = os.path.join(ROOT, "include")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          # packed fp32 instructions are not emitted (see the design notes)
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument"]

SOURCES = ["bd_api.cpp", "commit.hip", "lmhead.hip", "attn_fwd.hip", "attn_decode.hip", "attn_bwd.hip",
           "attn_f32.hip"]
# The decode kernel keeps its matrix accumulators in ordinary VGPRs (otherwise
# the compiler parks them in AGPRs and copies them back and forth every tile).
PER_FILE = {"attn_decode.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form=1"],
            "attn_bwd.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str, verbose: bool, build_dir: str, defines: dict) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *PER_FILE.get(src, []), *[f"-D{k}={v}" for k, v in defines.items()], "-c",
           os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if msg.strip() and verbose:
        print(msg, flush=True)
    return obj


def build(verbose: bool = False, defines: dict | None = None, lib_path: str | None = None,
          build_dir: str | None = None) -> str:
    """Compile all sources and link the library; returns its path.

    ``defines`` overrides the compile-time pipeline shapes (BD_DECODE_NS,
    BD_DECODE_TARGET_WGS); with ``lib_path`` the result is written
    elsewhere instead of replacing the package's libbd.so.
    """
    defines = dict(defines or {})
    build_dir = build_dir or BUILD
    lib_path = lib_path or LIB
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_dir, defines), SOURCES))
    tmp = lib_path + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
