"""Build the C-ABI example program (tests/c_abi/select_attend.c) with gcc.

    python tests/c_abi/build_example.py

A plain C11 program against include/qsa.h and the HIP runtime's C API,
linked to the in-tree libqsa.so (run path set to the package directory).
Built on the CPU host; the GPU test only runs it.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "sparse_attention_kv_qsa_amd")
SRC = os.path.join(HERE, "select_attend.c")
EXE = os.path.join(HERE, "select_attend")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(out: str = EXE, verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROCM}/include", f"-I{os.path.join(ROOT, 'include')}", SRC,
           f"-L{PKG}", "-lqsa", f"-L{ROCM}/lib", "-lamdhip64", "-lm",
           # $ORIGIN-relative run path: the package directory wherever the tree is
           "-Wl,-rpath,$ORIGIN/../../sparse_attention_kv_qsa_amd", f"-Wl,-rpath,{ROCM}/lib",
           "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
