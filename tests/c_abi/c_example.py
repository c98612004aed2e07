"""Build and run lynx_c_example.c, a plain C consumer of liblynx (C ABI and
HIP runtime only, no Python in the process).

    python -m tests.c_abi.c_example      # build tests/c_abi/lynx_c_example
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "lynx_c_example.c")
BIN = os.path.join(HERE, "lynx_c_example")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = True) -> str:
    """gcc, host code only; links liblynx.so (found next to the package at run
    time through an $ORIGIN-relative rpath) and the HIP runtime."""
    tmp = BIN + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-Werror",
           # the HIP runtime headers need the platform named when the compiler is not hipcc
           "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           SRC, "-o", tmp,
           "-L", os.path.join(ROOT, "activation_sparse_gemm_amd"), "-llynx",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../activation_sparse_gemm_amd",
           "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"gcc failed for {SRC}:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, BIN)
    if verbose:
        print(f"built {BIN}")
    return BIN


def run(args: list, timeout: float = 120.0) -> subprocess.CompletedProcess:
    if not os.path.exists(BIN):
        raise RuntimeError(f"{BIN} is missing: build it with `python -m tests.c_abi.c_example`")
    return subprocess.run([BIN, *map(str, args)], capture_output=True, text=True, timeout=timeout)


if __name__ == "__main__":
    build()
