"""Builds the HIP library ``libmoe_mi355x.so`` in-tree for gfx950.

Each ``csrc/*.hip`` file is compiled with hipcc into ``_build/`` (in
parallel), then linked into a shared library next to this file.  Packed fp32
instructions are switched off for the device code (``-packed-fp32-ops``).

The compiler's per-kernel resource report is kept in
``_build/resource_usage.json``; a kernel that spills registers to scratch
memory fails the build (every kernel here is sized to fit its registers).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import json
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe_mi355x.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _resource_usage(stderr: str) -> dict:
    """Kernel name -> {field: value} from -Rpass-analysis=kernel-resource-usage."""
    out, name = {}, None
    for line in stderr.splitlines():
        m = re.search(r"remark:\s+Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            out[name] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\d+)", line)
        if m and name:
            out[name][m.group(1).strip()] = int(m.group(2))
    return out


def _compile(src: str):
    obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj, _resource_usage(r.stderr)


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(SRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        done = list(ex.map(_compile, srcs))
    objs = [o for o, _ in done]
    usage = {k: v for _, u in done for k, v in u.items()}
    with open(os.path.join(OUT_DIR, "resource_usage.json"), "w") as f:
        json.dump(usage, f, indent=1, sort_keys=True)
    spills = {k: v.get("ScratchSize") for k, v in usage.items() if v.get("ScratchSize", 0) > 0}
    if spills:
        raise RuntimeError(f"kernels spill registers to scratch (bytes/lane): {spills}")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
