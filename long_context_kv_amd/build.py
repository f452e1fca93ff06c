"""Build libcartattn.so for gfx950 with hipcc (in-tree, no JIT cache).

Usage: python -m long_context_kv_amd.build [--jobs N] [--save-temps]

Every HIP translation unit is compiled with packed-fp32 instruction
generation disabled (those forms are avoided on this platform) and linked
into one shared library next to this file.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import pathlib
import subprocess
import sys

HERE = pathlib.Path(__file__).resolve().parent
ROOT = HERE.parent
CSRC = HERE / "csrc"
BUILD = HERE / "_build"
LIB = HERE / "libcartattn.so"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["cartattn.cpp", "timing.cpp", "rope.hip", "rows.hip", "attn_fwd.hip", "attn_bwd.hip",
           "decode.hip", "qknorm.hip", "adam.hip", "compose.hip"]

COMMON = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{ROOT / 'include'}",
    f"-I{CSRC}",
]


def _compile(src: pathlib.Path, save_temps: bool) -> pathlib.Path:
    obj = BUILD / (src.name + ".o")
    cmd = [HIPCC, *COMMON, "-c", str(src), "-o", str(obj)]
    if src.suffix == ".cpp":
        cmd[1:1] = ["-x", "hip"]
    if save_temps:
        cmd.append("-save-temps=obj")
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed on {src.name}")
    return obj


def build(jobs: int = 8, save_temps: bool = False) -> pathlib.Path:
    BUILD.mkdir(exist_ok=True)
    srcs = [CSRC / s for s in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, save_temps), srcs))
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", str(tmp),
           *map(str, objs)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("link of libcartattn.so failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=8)
    ap.add_argument("--save-temps", action="store_true")
    args = ap.parse_args()
    print(build(args.jobs, args.save_temps))
