"""Build the HQMQ HIP library for gfx950, in-tree.

    python -m kv_cache_quantization_hqmq_amd.build

compiles csrc/hqmq_kernels.hip, csrc/hqmq_search.hip, csrc/hqmq_attend.hip,
csrc/hqmq_ceiling.hip, csrc/hqmq_noalloc.hip and csrc/hqmq_api.cpp with hipcc
into kv_cache_quantization_hqmq_amd/libhqmq.so.  Every HIP translation unit is
built with packed FP32 disabled and fp contraction off (each fused
multiply-add in the kernels is written out).  hqmq_search.hip (the fp16-input
search) is also built with IEEE mode off and fp32 denormals flushed: the mode
in which the hardware applies VOP3 output modifiers (its file comment shows
why that mode changes none of its values).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libhqmq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall",
]
# kernels only (the host API validates floats and keeps IEEE semantics)
KERNEL_FLAGS = [
    # inputs are finite by contract: lets v_max/v_max3 take MFMA results
    # without canonicalising them first
    "-fno-honor-nans",
    # MFMA results in arch VGPRs (no v_accvgpr_read per result)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]
# per-file additions
FILE_FLAGS = {
    "hqmq_search.hip": ["-fgpu-flush-denormals-to-zero", "-mno-amdgpu-ieee"],
}
SOURCES = ("hqmq_kernels.hip", "hqmq_search.hip", "hqmq_attend.hip", "hqmq_ceiling.hip", "hqmq_noalloc.hip",
           "hqmq_api.cpp")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd[:3])} ...")
    # hipcc's host pass does not know the packed-fp32 feature: drop that noise
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if verbose and msg.strip():
        print(msg)


def build(verbose: bool = False) -> str:
    objs = []
    bdir = os.path.join(HERE, "_build")
    os.makedirs(bdir, exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(bdir, src + ".o")
        extra = ["-x", "hip", *KERNEL_FLAGS, *FILE_FLAGS.get(src, [])] if src.endswith(".hip") else []
        _run([HIPCC, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
