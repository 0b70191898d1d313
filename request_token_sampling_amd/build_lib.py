"""Build of the HIP library librts.so (gfx950), in-tree next to this file.

Run ``python -m request_token_sampling_amd.build_lib``.  Compiles every time
it is called (objects in request_token_sampling_amd/_build/).  Flags: -ffp-contract=off keeps the penalty arithmetic at one
rounding per operation; packed fp32 instructions are disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "librts.so")
SOURCES = ["rts_api.cpp", "rts_sample.hip", "rts_logprobs.hip", "rts_prior.hip", "rts_noalloc.hip"]
ARCH = os.environ.get("RTS_OFFLOAD_ARCH", "gfx950")
OBJ_DIR = os.path.join(HERE, "_build")

FLAGS = ["-O3", f"--offload-arch={ARCH}", "-std=c++17", "-fPIC", "-ffp-contract=off",
         "-fno-fast-math", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


def compile_cmd(src: str, obj: str) -> list:
    return ["/opt/rocm/bin/hipcc", *FLAGS, "-I", INCLUDE, "-I", CSRC, "-c",
            os.path.join(CSRC, src), "-o", obj]


def link_cmd(objs, out: str) -> list:
    return ["/opt/rocm/bin/hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out, *objs,
            "-Wl,-rpath,/opt/rocm/lib"]


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every source to an object (in parallel), then link librts.so."""
    from concurrent.futures import ThreadPoolExecutor

    os.makedirs(OBJ_DIR, exist_ok=True)
    objs = [os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o") for src in SOURCES]
    cmds = [compile_cmd(src, obj) for src, obj in zip(SOURCES, objs)]
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    n = jobs or min(len(cmds), max(1, min(os.cpu_count() or 1, 8)))
    with ThreadPoolExecutor(n) as pool:
        for rc, c in zip(pool.map(lambda c: subprocess.call(c), cmds), cmds):
            if rc != 0:
                raise subprocess.CalledProcessError(rc, c)
    tmp = LIB + ".tmp"
    cmd = link_cmd(objs, tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


CONSUMER_SRC = os.path.join(ROOT, "tests", "c_abi_consumer.cpp")
CONSUMER = os.path.join(ROOT, "tests", "_build", "c_abi_consumer")


def build_consumer(verbose: bool = False) -> str:
    """The plain C++ program in tests/ that uses the library through
    include/rts.h and the HIP runtime alone, linked to the in-tree librts.so."""
    os.makedirs(os.path.dirname(CONSUMER), exist_ok=True)
    tmp = CONSUMER + ".tmp"
    cmd = ["/opt/rocm/bin/hipcc", "-O2", "-std=c++17", "-Wall", "-I", INCLUDE, CONSUMER_SRC,
           "-o", tmp, "-L", HERE, "-lrts", "-Wl,-rpath,$ORIGIN/../../request_token_sampling_amd",
           "-Wl,-rpath,/opt/rocm/lib"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, CONSUMER)
    return CONSUMER


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_consumer(verbose=True))
    sys.exit(0)
