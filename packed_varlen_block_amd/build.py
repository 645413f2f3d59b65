"""Build libpvb.so (the C-ABI library) in-tree with hipcc for gfx950.

Usage: python -m packed_varlen_block_amd.build [--verbose] [--resource-usage] [--sanitize]
"""
from __future__ import annotations

import argparse
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libpvb.so")

SOURCES = ["abi.cpp", "pack_plan.cpp", "packed_row.hip", "packed_loss.hip", "attn_common.hip", "attn_fwd.hip",
           "attn_bwd.hip", "gated_delta.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed-fp32 VALU instructions are disabled for every HIP translation unit.
DEVICE_FLAGS = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON_FLAGS = ["-O3", "-fPIC", "-std=c++17", "-I" + INCLUDE, "-I" + CSRC, "-Wall", "-Wno-unused-function"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in r.stdout.splitlines()
                    if "packed-fp32-ops" not in line and line.strip())
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}")
    return out


# The CPU sanitizer build (libpvb_san.so): AddressSanitizer and
# UndefinedBehaviorSanitizer on the host code only (the planners, the ABI's
# argument checks, the launch set-up); the device code is built as usual.
# Every sanitizer flag is given to the host compilation alone.
SAN_LIB_PATH = os.path.join(HERE, "libpvb_san.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def build(verbose: bool = False, resource_usage: bool = False, jobs: int | None = None,
          sanitize: bool = False) -> str:
    bdir = BUILD_DIR + ("_san" if sanitize else "")
    os.makedirs(bdir, exist_ok=True)
    cmds, objs = [], []
    extra = SAN_FLAGS if sanitize else []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(bdir, src + ".o")
        cmd = [HIPCC, "-c", path, "-o", obj] + COMMON_FLAGS + extra
        if src.endswith(".hip"):
            cmd = [HIPCC, "-x", "hip", "-c", path, "-o", obj] + COMMON_FLAGS + DEVICE_FLAGS + extra
            if resource_usage:
                cmd += ["-Rpass-analysis=kernel-resource-usage"]
        cmds.append(cmd)
        objs.append(obj)
    # one compiler process per source, at most `jobs` at a time
    n = jobs or min(len(cmds), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(max_workers=n) as ex:
        for out in ex.map(lambda c: _run(c, verbose), cmds):
            if out and (verbose or resource_usage):
                print(out)
    lib_path = SAN_LIB_PATH if sanitize else LIB_PATH
    tmp = lib_path + ".tmp"
    _run([HIPCC, "-shared", "-o", tmp] + objs + ["--offload-arch=" + ARCH] + extra, verbose)
    os.replace(tmp, lib_path)
    return lib_path


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--resource-usage", action="store_true")
    ap.add_argument("--sanitize", action="store_true",
                    help="build libpvb_san.so with host AddressSanitizer and UBSan (CPU checks)")
    a = ap.parse_args(argv)
    print(build(a.verbose, a.resource_usage, sanitize=a.sanitize))


if __name__ == "__main__":
    sys.exit(main())
