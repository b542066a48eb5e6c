"""Build libbacklite.so (the HIP kernels + C ABI) in-tree for gfx950.

    python -m block_sparse_attention_fa_amd.build

Every .hip file under csrc/ is compiled by hipcc for gfx950, and every .cpp
file (host-only C++) by the host compiler, to an object under _build/ (in
parallel); the objects are linked into block_sparse_attention_fa_amd/libbacklite.so.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libbacklite.so")
ROOT = os.path.dirname(PKG)

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # no packed fp32 arithmetic in device code (v_pk_* f32 forms)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics", "-Wno-unused-command-line-argument",
    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
]


# per-file extra flags: the G_Q pass keeps MFMA results in arithmetic registers
# (its S / G_P accumulators feed VALU work; measured 11% faster on MI355X),
# while the G_K/G_V pass keeps its accumulators in AGPRs: with arithmetic-
# register results its 128 long-lived G_K/G_V accumulators plus the S / G_P
# chunks exceed the 256 VGPRs and spill.
FILE_FLAGS = {"bwd_dq.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libbacklite.so)")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


HOST_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-Wall", f"-I{os.path.join(ROOT, 'include')}"]


def host_cxx() -> str:
    for c in (os.environ.get("CXX"), shutil.which("g++"), shutil.which("c++")):
        if c and shutil.which(c):
            return c
    raise RuntimeError("no host C++ compiler found")


def build(verbose: bool = False, incremental: bool = False) -> str:
    """Compile and link.  incremental=True (development only) skips sources
    whose object is newer than the source and every header."""
    cc = hipcc()
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))
    objs = [os.path.join(BUILD, os.path.splitext(f)[0] + ".o") for f in srcs]
    hdr_time = max([os.path.getmtime(os.path.join(d, f)) for d in (CSRC, os.path.join(ROOT, "include"))
                    for f in os.listdir(d) if f.endswith(".h")] or [0.0])

    def comp(i):
        if incremental and os.path.exists(objs[i]) and os.path.getmtime(objs[i]) > max(
                hdr_time, os.path.getmtime(os.path.join(CSRC, srcs[i]))):
            return ""
        src = os.path.join(CSRC, srcs[i])
        if srcs[i].endswith(".cpp"):
            return _run([host_cxx(), *HOST_FLAGS, "-c", src, "-o", objs[i]])
        return _run([cc, *FLAGS, *FILE_FLAGS.get(srcs[i], []), "-c", src, "-o", objs[i]])

    jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with ThreadPoolExecutor(jobs) as ex:
        outs = list(ex.map(comp, range(len(srcs))))
    tmp = LIB + ".tmp"
    outs.append(_run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]))
    os.replace(tmp, LIB)
    if verbose:
        for o in outs:
            if o:
                print(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, incremental="--incremental" in sys.argv))
    sys.exit(0)
