"""Build libpkv.so in-tree: the HIP kernels for gfx950 plus the host allocator.

Run `python -m paged_kv_cache_387_amd.build` (or `__graft_entry__.build()`).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libpkv.so")
OBJ_DIR = os.path.join(HERE, "_build")

HIP_SOURCES = ["api.hip", "decode.hip", "decode_runs.hip", "decode_stream.hip", "prefix.hip",
               "prefix_pipe.hip",
               "cache_ops.hip"]
CXX_SOURCES = ["allocator.cpp"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in the generated code.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I" + INCLUDE,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function"]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-I" + INCLUDE]
# The multi-query passes keep their accumulators, q and scores in the unified
# register file: with the MFMA results in VGPRs (the instruction's VGPR form)
# the softmax reads the scores without a copy per element, and the quantized
# passes fit without scratch.  The decode kernels hold no AGPRs either way.
SOURCE_FLAGS = {src: ["-mllvm", "-amdgpu-mfma-vgpr-form"]
                for src in ("prefix.hip", "prefix_pipe.hip")}


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return res


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(OBJ_DIR, src + ".o")
        jobs.append([HIPCC, *HIP_FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src),
                     "-o", obj])
    for src in CXX_SOURCES:
        obj = os.path.join(OBJ_DIR, src + ".o")
        jobs.append(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for res in ex.map(_run, jobs):
            if verbose and res.stderr:
                sys.stderr.write(res.stderr)
    objs = [os.path.join(OBJ_DIR, s + ".o") for s in HIP_SOURCES + CXX_SOURCES]
    tmp = LIB + f".tmp{os.getpid()}"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
