"""Host AddressSanitizer + UndefinedBehaviorSanitizer run of the CPU suite.

    python tests/sanitize_host.py [extra pytest args]

Builds, with clang's sanitizers on the host code only:

  * the oracle (oracle/hqmq_oracle.c) -> tests/_san/libhqmq_oracle_san.so,
    single-threaded (no OpenMP, so one sanitizer runtime sees every access);
  * the library -> tests/_san/libhqmq_san.so: every translation unit of
    kv_cache_quantization_hqmq_amd/build.py with the same flags plus
    -fsanitize=address,undefined on the host side (-Xarch_host); the gfx950
    device code is built as usual and is not run here;

then runs ``pytest -m "not gpu"`` with the sanitizer runtime preloaded and
HQMQ_LIB / HQMQ_ORACLE_LIB pointing at the two builds.  Any report aborts
the run (halt_on_error, no recovery), so exit status 0 means the suite passed
with zero reports.  Leak checking is off (the interpreter keeps allocations
until exit); allocation/deallocation-mismatch and ODR checks are off for the
uninstrumented libraries the interpreter loads (torch).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)

from kv_cache_quantization_hqmq_amd import build as B  # noqa: E402

OUT = os.path.join(HERE, "_san")
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def runtime() -> str:
    libs = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not libs:
        raise RuntimeError("clang's AddressSanitizer runtime is not installed")
    return libs[0]


def build_oracle() -> str:
    out = os.path.join(OUT, "libhqmq_oracle_san.so")
    src = os.path.join(ROOT, "oracle", "hqmq_oracle.c")
    cmd = [CLANG, "-O1", "-std=gnu11", "-ffp-contract=off", "-fno-fast-math", "-Wno-unknown-pragmas",
           "-shared", "-fPIC", "-shared-libasan", *SAN, src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def build_library() -> str:
    out = os.path.join(OUT, "libhqmq_san.so")
    host = [f for s in SAN for f in ("-Xarch_host", s)]
    objs = []
    for src in B.SOURCES:
        obj = os.path.join(OUT, src + ".o")
        extra = ["-x", "hip", *B.KERNEL_FLAGS, *B.FILE_FLAGS.get(src, []), *host] if src.endswith(".hip") else SAN
        B._run([B.HIPCC, *B.COMMON, *extra, "-c", os.path.join(B.CSRC, src), "-o", obj], False)
        objs.append(obj)
    B._run([B.HIPCC, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-shared-libasan", *SAN, *objs, "-o", out],
           False)
    return out


def main(argv) -> int:
    os.makedirs(OUT, exist_ok=True)
    print("building the sanitized oracle and library ...", flush=True)
    oracle_lib = build_oracle()
    hqmq_lib = build_library()
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": runtime(),
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:alloc_dealloc_mismatch=0:detect_odr_violation=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "HQMQ_LIB": hqmq_lib,
        "HQMQ_ORACLE_LIB": oracle_lib,
    })
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-m", "not gpu", "-x", "-q",
           "-p", "no:cacheprovider", *argv]
    print(" ".join(cmd), flush=True)
    return subprocess.run(cmd, cwd=ROOT, env=env).returncode


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
