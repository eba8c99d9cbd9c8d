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
import re
import subprocess
import sys
import tempfile

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


def _llvm_tool(name: str) -> str:
    base = os.path.dirname(os.path.realpath(_hipcc()))
    for cand in (os.path.join(base, "..", "lib", "llvm", "bin", name), os.path.join(base, "..", "llvm", "bin", name),
                 os.path.join("/opt/rocm/lib/llvm/bin", name), shutil.which(name)):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError(f"{name} not found")


_THIN = re.compile(r"<(_Z\S*gemm_kernelILi\d+ELi\d+ELb(\d)ELi1ELi(\d)ELb(\d)E\S*)>:")
_META = ("global_load_ushort", "global_load_short_d16", "global_load_dword", "global_load_sshort")


def check_thin_tile_waits(obj: str) -> int:
    """The 32-token GEMM tiles keep the step after next in flight across the
    step barrier with a partial wait, vmcnt(WP * CB + 2): that count is right
    only if the last vector memory instructions before the barrier are that
    step's WP * CB 16-byte weight loads and two x loads into LDS (its
    metadata before them).  Checks it in the disassembly of this build's own
    gfx950 code (one object file); returns the number of barriers checked,
    raises if one breaks it."""
    with tempfile.TemporaryDirectory() as d:
        fat, co = os.path.join(d, "fatbin"), os.path.join(d, "code.o")
        for cmd in ([_llvm_tool("llvm-objcopy"), f"--dump-section=.hip_fatbin={fat}", obj, os.path.join(d, "host.o")],
                    [_llvm_tool("clang-offload-bundler"), "--type=o", f"--targets=hipv4-amdgcn-amd-amdhsa--{ARCH}",
                     f"--input={fat}", f"--output={co}", "--unbundle"]):
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"{cmd[0]} failed:\n{r.stderr}")
        r = subprocess.run([_llvm_tool("llvm-objdump"), "-d", f"--mcpu={ARCH}", co], capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"llvm-objdump failed:\n{r.stderr}")
    return thin_tile_waits_in(r.stdout)


def thin_tile_waits_in(disassembly: str) -> int:
    """The check of check_thin_tile_waits on llvm-objdump text."""
    checked, kernel, keep, wpcb, meta_first, vm, prev = 0, None, 0, 0, False, [], ""
    for line in disassembly.splitlines():
        m = _THIN.search(line)
        if m:
            cb, dense = int(m.group(3)), m.group(4) == "1"
            kernel, wpcb, vm, prev = m.group(1), (8 if dense else 2) * cb, [], ""
            keep, meta_first = wpcb + 2, not dense
            continue
        if line.endswith(">:"):
            kernel = None
            continue
        if kernel is None or not line.startswith("\t"):
            continue
        ins = line.strip().split("//")[0].strip()
        op = ins.split(" ")[0]
        if op.startswith(("global_", "buffer_")):
            vm.append(op)
        elif op == "s_barrier":
            w = re.match(r"s_waitcnt vmcnt\((\d+)\)", prev)
            if w and int(w.group(1)) > 0:
                n = int(w.group(1))
                want = ["global_load_dwordx4"] * wpcb + ["global_load_lds_dwordx4"] * 2
                ok = n == keep and vm[-n:] == want and (not meta_first or (len(vm) > n and vm[-n - 1] in _META))
                if not ok:
                    raise RuntimeError(f"{kernel}: '{prev}' before a step barrier, but the last vector memory "
                                       f"instructions are {vm[-(n + 1):]}")
                checked += 1
            vm = []
        prev = ins
    return checked


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
    # the thin GEMM tiles' partial wait relies on the compiled load order
    if check_thin_tile_waits(objs[SOURCES.index("w4a16_gemm.hip")]) == 0:
        raise RuntimeError("no partial-wait step barrier found in the 32-token GEMM tiles")
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], CEILINGS_LIB)
    if verbose:
        print(f"built {LIB} and {CEILINGS_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
