"""Register guard for the HIP kernels (CPU only: a device-only compile).

Every kernel of the library is compiled for gfx950 with the compiler's
per-kernel resource remarks (-Rpass-analysis=kernel-resource-usage), and the
test fails if any kernel spills vector registers or uses scratch memory: a
kernel that starts spilling after a change runs at a fraction of its speed
without any other sign.  Scalar-register spills (to lanes of a vector
register, no memory traffic) are listed but not failed.

Run with -s to print the table of VGPRs, AGPRs, SGPRs, spills, scratch, LDS
and occupancy of every kernel.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_attention_kv_qsa_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FIELDS = {
    "VGPRs": "vgpr", "AGPRs": "agpr", "TotalSGPRs": "sgpr", "ScratchSize [bytes/lane]": "scratch",
    "Occupancy [waves/SIMD]": "occupancy", "SGPRs Spill": "sgpr_spill",
    "VGPRs Spill": "vgpr_spill", "LDS Size [bytes/block]": "lds",
}


def compile_remarks(path: str, outdir: str) -> list[dict]:
    from sparse_attention_kv_qsa_amd.build import ARCH, flags_for
    flags = flags_for(path)
    cmd = [HIPCC, *flags, f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", "-c", path,
           "--offload-device-only", "-Rpass-analysis=kernel-resource-usage",
           "-o", os.path.join(outdir, os.path.basename(path) + ".o")]
    assert f"--offload-arch={ARCH}" in cmd
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    rows, cur = [], None
    for line in r.stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = {"file": os.path.basename(path), "symbol": m.group(1)}
            rows.append(cur)
            continue
        m = re.search(r"remark:\s+(.+?): (\S+) \[-Rpass-analysis", line)
        if m and cur is not None and m.group(1) in FIELDS:
            val = m.group(2)
            cur[FIELDS[m.group(1)]] = int(val) if val.isdigit() else val
    return rows


@pytest.fixture(scope="module")
def kernels():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    d = tempfile.mkdtemp()
    try:
        with cf.ThreadPoolExecutor(len(srcs)) as ex:
            rows = [r for rs in ex.map(lambda p: compile_remarks(p, d), srcs) for r in rs]
    finally:
        shutil.rmtree(d, ignore_errors=True)
    names = subprocess.run(["c++filt"], input="\n".join(r["symbol"] for r in rows),
                           capture_output=True, text=True).stdout.splitlines()
    for r, n in zip(rows, names):
        n = n.replace("qsa::(anonymous namespace)::", "")
        r["name"] = re.sub(r"^void ", "", re.sub(r"\(.*\)$", "", n))
    print("\n" + "\n".join(
        f"{r['file']:24s} {r['name']:46s} VGPR {r.get('vgpr', '?'):>3} AGPR {r.get('agpr', '?'):>3} "
        f"SGPR {r.get('sgpr', '?'):>3} spill V/S {r.get('vgpr_spill', '?')}/{r.get('sgpr_spill', '?')} "
        f"scratch {r.get('scratch', '?'):>3} LDS {r.get('lds', '?'):>6} occ {r.get('occupancy', '?')}"
        for r in rows))
    return rows


def test_every_kernel_reports(kernels):
    names = {r["name"].split("<")[0] for r in kernels}
    for k in ("scores_bf16x3_kernel", "scores_f16x2_kernel", "scores_mfma_kernel", "scores_gemv_kernel",
              "scores_gemv_tops_kernel", "topk_kernel", "group_tops_kernel", "wide_rank_kernel",
              "attn_chunk_kernel", "attn_chunk_i8_kernel", "attn_merge_kernel"):
        assert k in names, f"no resource remarks for {k}"
    for r in kernels:
        assert "vgpr_spill" in r and "scratch" in r, r


def test_no_vector_spills_or_scratch(kernels):
    bad = [f"{r['name']}: {r['vgpr_spill']} VGPRs spilled, {r['scratch']} B/lane scratch"
           for r in kernels if r["vgpr_spill"] != 0 or r["scratch"] != 0]
    assert not bad, "kernels spilling to scratch:\n" + "\n".join(bad)
