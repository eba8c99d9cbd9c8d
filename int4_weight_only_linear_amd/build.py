"""Build libw4a16.so in-tree for gfx950 with hipcc.

    python -m int4_weight_only_linear_amd.build        # or: from ... import build; build()

Every translation unit is compiled in parallel to an object under ``_build/``
and linked into ``int4_weight_only_linear_amd/libw4a16.so``.  All device
code is compiled without packed-fp32 instruction selection; the decode kernels
with kernel-argument preloading.
"""
from __future__ import annotations

import concurrent.futures as cf
import json
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libw4a16.so")

ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
SOURCES = ["w4a16_host.cpp", "w4a16_gemv.hip", "w4a16_gemm.hip", "w4a16_elementwise.hip"]
# measurement kernels for the benchmark's ceilings, a library of their own
CEILING_SOURCES = ["w4a16_ceilings.hip"]
CEILINGS_LIB = os.path.join(PKG, "libw4a16_ceilings.so")
# the decode kernel takes its first ten arguments preloaded into SGPRs
EXTRA = {"w4a16_gemv.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=10"]}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; libw4a16 needs ROCm's hipcc to build")


_REMARK = "kernel-resource-usage"


def _resources(text: str) -> dict:
    """Per-kernel register use from hipcc's resource-usage remarks."""
    res, name = {}, None
    for line in text.splitlines():
        if _REMARK not in line or "remark:" not in line:
            continue
        body = line.split("remark:", 1)[1].split("[-R", 1)[0].strip()
        key, _, val = body.partition(":")
        if key == "Function Name":
            name = val.strip()
            res[name] = {}
        elif name is not None and val.strip().lstrip("-").isdigit():
            res[name][key.strip()] = int(val)
    return res


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *COMMON, *EXTRA.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd.append(f"-Rpass-analysis={_REMARK}")
    r = subprocess.run(cmd, capture_output=True, text=True)
    text = r.stdout + r.stderr
    out = "\n".join(l for l in text.splitlines()
                    if "packed-fp32-ops" not in l and _REMARK not in l and not l.lstrip().startswith(("|", "^"))
                    and not l.lstrip()[:1].isdigit())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{text}")
    if src.endswith(".hip"):
        # register and scratch use of every kernel instance, kept beside the
        # object (the GEMM planner's tile table is checked against it)
        with open(obj + ".resources.json", "w") as f:
            json.dump(_resources(text), f, indent=1, sort_keys=True)
    if out.strip():
        print(out, file=sys.stderr)
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile and link libw4a16.so (and the benchmark's ceiling kernels,
    libw4a16_ceilings.so); returns the path of libw4a16.so."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + len(CEILING_SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES + CEILING_SOURCES))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], CEILINGS_LIB)
    if verbose:
        print(f"built {LIB} and {CEILINGS_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
