"""Build librq.so (the C-ABI HIP library) in-tree for gfx950.

    python -m looped_transformer_kv_rq_amd.build

Every .hip source under csrc/ is compiled by hipcc (in parallel) into
_build/, then linked into looped_transformer_kv_rq_amd/librq.so.
"""
from __future__ import annotations

import glob
import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "librq.so")
ARCH = "gfx950"

CXXFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU ops stay off on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature; drop that noise
    out = "\n".join(l for l in proc.stdout.splitlines() if "packed-fp32-ops" not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    return out


def scratch_users(log: str) -> list:
    """(kernel, bytes per lane) of every kernel whose resource-usage remark in
    a compile log reports private (scratch) memory, i.e. register spills."""
    out, name = [], None
    for line in log.splitlines():
        m = re.search(r"remark:\s+Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name is not None and int(m.group(1)) > 0:
            out.append((name, int(m.group(1))))
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(BUILD, os.path.basename(s) + ".o") for s in sources]

    def compile_one(pair):
        src, obj = pair
        return _run([cc, *CXXFLAGS, "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj])

    with ThreadPoolExecutor(max(1, min(8, len(sources)))) as ex:
        logs = list(ex.map(compile_one, zip(sources, objs)))
    # No kernel may spill registers to scratch: builds of the 128-coordinate
    # INT3 / INT8 decode kernel whose register allocation spilled gave wrong
    # attention rows on MI355X (every spill-free build of the same source was
    # correct), so a spill fails the build instead of shipping.
    spills = [u for log in logs for u in scratch_users(log)]
    if spills:
        raise RuntimeError("kernels spill registers to scratch: " + ", ".join(f"{k} ({n} B/lane)" for k, n in spills))
    logs = ["\n".join(x for x in log.splitlines() if "remark:" not in x) for log in logs]
    tmp = LIB + ".tmp"
    logs.append(_run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs,
                      "-Wl,-rpath,/opt/rocm/lib"]))
    os.replace(tmp, LIB)
    if verbose:
        for l in logs:
            if l.strip():
                print(l)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
