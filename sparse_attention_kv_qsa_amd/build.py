"""Build libqsa.so for gfx950 with hipcc (in-tree, next to this file).

    python -m sparse_attention_kv_qsa_amd.build

Cross-compiles on a host without a GPU.  Packed-fp32 instructions are switched
off for all device code (``-Xclang -target-feature -Xclang -packed-fp32-ops``);
hipcc's host pass warns that it does not know that feature, which is harmless.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libqsa.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]

# The instruction scheduler's maximum-ILP strategy, for the scoring and
# selection sources: every select call timed faster with it or unchanged
# (scorer 64.8 -> 64.0 us on 256 x 32K blocks, decode select 19.9 -> 19.7 us,
# near-tie top-k 37.8 -> 37.0 us; same box, outputs bitwise equal), with no
# spill in any kernel.  The attention kernels keep the default schedule:
# against it their calls moved by -1.1 to +0.2 us depending on the case (fp32
# at k = 4096 slower in every run), no consistent gain.
SCHED_MAX_ILP = ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]
DEFAULT_SCHEDULE = {"qsa_attn.hip"}


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def flags_for(path: str) -> list[str]:
    """Compiler flags of one source file (without -c / -shared / -o)."""
    sched = [] if os.path.basename(path) in DEFAULT_SCHEDULE else SCHED_MAX_ILP
    return [*HIPCC_FLAGS, *sched]


def build(verbose: bool = False, extra: list[str] | None = None, out: str = LIB_PATH) -> str:
    """Compile every csrc/*.hip (one object each, in parallel: every file's
    device code is self-contained) and link them into one shared library;
    returns its path."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp"
    with tempfile.TemporaryDirectory() as objdir:
        cmds = []
        for src in sources():
            obj = os.path.join(objdir, os.path.basename(src) + ".o")
            cmds.append(([hipcc, *flags_for(src), *(extra or []), f"-I{INCLUDE}", f"-I{CSRC}",
                          "-c", src, "-o", obj], obj))
        procs = []
        for cmd, _ in cmds:
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append(subprocess.Popen(cmd))
        failed = [cmd for (cmd, _), p in zip(cmds, procs) if p.wait() != 0]
        if failed:
            raise subprocess.CalledProcessError(1, failed[0])
        link = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *(obj for _, obj in cmds),
                "-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        subprocess.run(link, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True, extra=sys.argv[1:]))
