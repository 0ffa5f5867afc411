"""Build libslimkv.so (HIP, gfx950) in-tree.

    python -m latent_decode_attention_amd.build [--verbose] [--resource-usage]

Compiles every source under csrc/ with hipcc in parallel into _build/ at the
repository root and links latent_decode_attention_amd/libslimkv.so.  Always
rebuilds.  ``--resource-usage`` prints each kernel's VGPR/SGPR/LDS use and
occupancy as reported by the compiler.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import pathlib
import shutil
import subprocess
import sys

PKG = pathlib.Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
BUILD = ROOT / "_build"
LIBRARY = PKG / "libslimkv.so"
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def compile_flags(resource_usage: bool = False) -> list:
    flags = [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Wall", "-Wno-unused-function",
        # no packed-fp32 instructions in device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        f"-I{INCLUDE}", f"-I{CSRC}",
    ]
    if resource_usage:
        flags.append("-Rpass-analysis=kernel-resource-usage")
    return flags


def _compile(src: pathlib.Path, flags: list, verbose: bool) -> pathlib.Path:
    obj = BUILD / (src.name + ".o")
    cmd = [hipcc(), *flags, "-c", str(src), "-o", str(obj)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in res.stderr.splitlines() if noise not in line)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {src.name}\n{err}")
    if verbose and err.strip():
        print(f"--- {src.name}\n{err}", file=sys.stderr)
    return obj


def build(verbose: bool = False, resource_usage: bool = False, jobs: int | None = None) -> pathlib.Path:
    BUILD.mkdir(exist_ok=True)
    sources = sorted(CSRC.glob("*.hip")) + sorted(CSRC.glob("*.cpp"))
    flags = compile_flags(resource_usage)
    jobs = jobs or min(8, os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, flags, verbose or resource_usage), sources))
    tmp = LIBRARY.with_suffix(".so.tmp")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed\n{res.stderr}")
    os.replace(tmp, LIBRARY)
    return LIBRARY


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--resource-usage", action="store_true")
    args = ap.parse_args()
    print(build(verbose=args.verbose, resource_usage=args.resource_usage))


if __name__ == "__main__":
    main()
