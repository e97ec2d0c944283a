"""Build libnvfp4.so (HIP, gfx950) in place, next to this file.

    python -m nvfp4_moe_expert_amd.build

The library is plain hipcc output: every .hip under csrc/ is compiled for
gfx950 and linked into one shared object with a C ABI (include/nvfp4.h).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libnvfp4.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # bit-reproducible arithmetic: no FMA contraction, IEEE division (hipcc default)
    "-ffp-contract=off",
    # packed-fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(msgs))
    if msgs:
        print("\n".join(msgs), file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    """Compile every csrc/*.hip for gfx950 and link libnvfp4.so. Always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
