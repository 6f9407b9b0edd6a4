"""Build libqdecode.so in-tree for gfx950 with hipcc.

Every .hip file under csrc/ is compiled to an object (in parallel), then the
objects are linked into ``quantized_transformer_decode_amd/libqdecode.so``.
The quantize kernel is compiled with -ffp-contract=off (its encoding must
match ggml's f32 rounding bit for bit).  The prefill GEMM keeps its MFMA
results in ordinary VGPRs (fewer registers than the AGPR form, so two
workgroups fit per CU).  Packed-fp32 VALU instructions are disabled for all
device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libqdecode.so")
OBJDIR = os.path.join(HERE, "_build")

ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-Wall", "-Wno-unused-command-line-argument",
]
PER_FILE = {
    "q4_0_quantize.hip": ["-ffp-contract=off"],
    "q4_0_gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(OBJDIR, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(OBJDIR, src[:-4] + ".o")
        cmd = [hipcc, *COMMON, *PER_FILE.get(src, []), "-c",
               os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr, file=sys.stderr)
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, sources()))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc, "-shared", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
