"""Build libtl.so in-tree for gfx950 with hipcc.

    python -m tl_hadamard_rotate_amd.build          # compile every csrc/*.hip

Objects go to tl_hadamard_rotate_amd/_build/, the library to
tl_hadamard_rotate_amd/libtl.so (both git-ignored).  The benchmark's
read-only probe (probe/*.hip) becomes a library of its own,
libtl_probe.so, so that it is not part of the layer library.  Always
recompiles.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
PROBE = os.path.join(PKG, "probe")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libtl.so")
PROBE_LIB = os.path.join(PKG, "libtl_probe.so")
ARCH = "gfx950"

# packed fp32 VALU instructions are kept out of the generated code
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libtl)")


def sources(folder: str = CSRC) -> list[str]:
    return sorted(os.path.join(folder, f) for f in os.listdir(folder) if f.endswith(".hip"))


def _compile(src: str) -> str:
    sub = os.path.basename(os.path.dirname(src))
    obj = os.path.join(BUILD, sub + "_" + os.path.basename(src)[:-4] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def _link(objs: list[str], lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs, probes = sources(CSRC), sources(PROBE)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs) + len(probes))) as ex:
        objs = list(ex.map(_compile, srcs + probes))
    _link(objs[:len(srcs)], LIB)
    _link(objs[len(srcs):], PROBE_LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources and {PROBE_LIB} from {len(probes)}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
