"""Build the gfx950 HIP library libdsa_amd.so in-tree with hipcc (no JIT, no torch extension).

    python -m dsa_indexer_top_key_amd.build [--remarks]

Each source is compiled to an object under _build/ in parallel and linked into
dsa_indexer_top_key_amd/libdsa_amd.so.  Every HIP source is compiled with packed-fp32
instructions disabled.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdsa_amd.so")
SOURCES = ["ln_keys.hip", "indexer.hip", "indexer_prefill.hip", "topk.hip", "sparse_mla.hip", "value_gate.hip",
           "indexer_proj.hip", "indexer_fp8.hip", "dsa_api.cpp"]
# Per-file code-generation options.  sparse_mla: MFMA results in VGPRs where they fit (its
# output accumulators then stay put; with the default AGPR form the register allocator
# shuttled one output tile between AGPRs and VGPRs around every S^T chain).
# indexer_prefill: same reason -- its VALU epilogue reads every accumulator, which from AGPRs
# would cost one extra move per value.
EXTRA_FLAGS = {"sparse_mla.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
               "indexer_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the DSA library)")


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function"]


def compile_one(src: str, remarks: bool) -> tuple[str, str]:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *common_flags(), *EXTRA_FLAGS.get(src, []), "-x", "hip", "-c",
           os.path.join(CSRC, src), "-o", obj]
    if remarks:
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj, r.stderr


def build(remarks: bool = False, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        results = list(ex.map(lambda s: compile_one(s, remarks), SOURCES))
    objs = [o for o, _ in results]
    if verbose or remarks:
        for _, log in results:
            if log.strip():
                print(log)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(remarks="--remarks" in sys.argv, verbose=True))
