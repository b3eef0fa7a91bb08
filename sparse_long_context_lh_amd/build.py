"""Build liblh.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m sparse_long_context_lh_amd.build [--jobs N]

Every source under csrc/ is compiled with hipcc to its own object (in
parallel), then linked into sparse_long_context_lh_amd/liblh.so.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "liblh.so")
SOURCES = ["lh_api.hip", "lh_front.hip", "lh_select.hip", "lh_gather.hip", "lh_attn.hip", "lh_scatter.hip",
           "lh_layer.hip"]
# rocBLAS runs the projection GEMMs of the step around the layer (lh_layer.hip)
LIBS = ["-L/opt/rocm/lib", "-lrocblas", "-Wl,-rpath,/opt/rocm/lib"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-Wall", "-Wno-unused-function",
    # packed fp32 VALU ops stay off: hipcc must not emit v_pk_{add,mul,fma}_f32.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# Per-source additions. The attention kernels keep their MFMA accumulators in
# ordinary VGPRs where they fit: the vector work on logits and outputs then
# reads them directly instead of copying out of accumulation registers.
EXTRA = {"lh_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def source_digest() -> str:
    """SHA-256 over the compiler flags and every source and header under csrc/ and include/."""
    h = hashlib.sha256()
    h.update(repr((FLAGS, EXTRA)).encode())
    inc = os.path.join(os.path.dirname(HERE), "include")
    for d in (CSRC, inc):
        for name in sorted(os.listdir(d)):
            h.update(name.encode())
            with open(os.path.join(d, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s\n%s" % (src, " ".join(cmd), res.stderr))
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in res.stderr.splitlines() if ln.strip() and noise not in ln]
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def build_library(jobs: int | None = None) -> str:
    """Compile every source and link liblh.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "--offload-arch=gfx950", *objs, *LIBS, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), res.stderr))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    print(build_library(ap.parse_args().jobs))
