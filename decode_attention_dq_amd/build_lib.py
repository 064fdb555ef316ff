"""Build libdq.so (the HIP kernels and their C ABI) in place for gfx950.

    python -m decode_attention_dq_amd.build_lib [--jobs N]

Each translation unit is compiled by hipcc for gfx950 only; the cache-write
unit is compiled without floating-point contraction so that its fp64
arithmetic is exactly the operation sequence written in the source.
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libdq.so")
BUILD = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["-std=c++17", "-O3", "-fPIC", "--offload-arch=gfx950", f"-I{INCLUDE}", f"-I{CSRC}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall", "-Wno-unused-function"]
UNITS = {
    "dq_api.cpp": [],
    "dq_attn.hip": [],
    "dq_bf16.hip": [],
    "dq_merge.hip": [],
    "dq_window.hip": [],
    "dq_token_attn.hip": [],
    "dq_encode.hip": ["-ffp-contract=off"],
}


def _compile(name: str) -> str:
    src = os.path.join(CSRC, name)
    obj = os.path.join(BUILD, name + ".o")
    cmd = [HIPCC, *COMMON, *UNITS[name], "-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {name}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 3) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, UNITS))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    return OUT


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=3)
    args = ap.parse_args()
    print(build(args.jobs))


if __name__ == "__main__":
    sys.exit(main())
