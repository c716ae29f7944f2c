"""The C ABI without a GPU: the library loads, exports what include/qsa.h
declares, and rejects bad arguments before touching the HIP runtime."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

from sparse_attention_kv_qsa_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qsa.h")


def header_entry_points() -> list[str]:
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qsa_[a-z0-9_]+)\s*\(", text)))


def header_macros() -> dict[str, int]:
    return {m: int(v) for m, v in re.findall(r"#define\s+(QSA_[A-Z0-9_]+)\s+(\d+)", open(HEADER).read())}


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.library_path()):
        pytest.fail("libqsa.so is not built (run __graft_entry__.build())")
    return binding.load_library()


def test_header_declares_the_entry_points():
    assert header_entry_points() == ["qsa_block_scores", "qsa_block_scores_ex", "qsa_block_select",
                                     "qsa_block_select_noalloc",
                                     "qsa_block_topk", "qsa_sparse_decode_attention",
                                     "qsa_sparse_decode_attention_i8", "qsa_strerror"]


def test_binding_covers_the_header():
    assert sorted(binding.SIGNATURES) == header_entry_points()
    mac = header_macros()
    assert (mac["QSA_OK"], mac["QSA_ERR_NULL"], mac["QSA_ERR_SHAPE"], mac["QSA_ERR_K"],
            mac["QSA_ERR_ALIGN"], mac["QSA_ERR_LAUNCH"]) == (
        binding.QSA_OK, binding.QSA_ERR_NULL, binding.QSA_ERR_SHAPE, binding.QSA_ERR_K,
        binding.QSA_ERR_ALIGN, binding.QSA_ERR_LAUNCH)
    assert mac["QSA_TOPK_MAX_K"] == binding.TOPK_MAX_K
    assert mac["QSA_MAX_ACTIVE_BLOCKS"] == binding.MAX_ACTIVE_BLOCKS
    assert mac["QSA_TOPK_FEW_ROWS"] == binding.TOPK_FEW_ROWS
    assert mac["QSA_ERR_MODE"] == binding.QSA_ERR_MODE
    assert mac["QSA_ERR_NOMEM"] == binding.QSA_ERR_NOMEM
    assert mac["QSA_ERR_SCRATCH"] == binding.QSA_ERR_SCRATCH
    assert mac["QSA_NOALLOC_SCRATCH_BYTES"] == binding.QSA_NOALLOC_SCRATCH_BYTES
    assert (mac["QSA_SCORES_AUTO"], mac["QSA_SCORES_FP32"], mac["QSA_SCORES_BF16X3"],
            mac["QSA_SCORES_F16X2"]) == (binding.QSA_SCORES_AUTO, binding.QSA_SCORES_FP32,
                                         binding.QSA_SCORES_BF16X3, binding.QSA_SCORES_F16X2)
    assert mac["QSA_MAX_HEAD_DIM"] == binding.QSA_MAX_HEAD_DIM
    assert mac["QSA_ATTN_MAX_DIM"] == binding.QSA_ATTN_MAX_DIM


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", binding.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (qsa_[a-z0-9_]+)$", out, flags=re.M))
    for name in header_entry_points():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_library_is_built_for_gfx950_only():
    # The offload bundle of our own build names its code-object targets.
    data = open(binding.library_path(), "rb").read()
    targets = set(re.findall(rb"amdgcn-amd-amdhsa-+(gfx[0-9a-z]+)", data))
    assert targets == {b"gfx950"}, targets


def test_strerror(lib):
    for code in range(9):
        assert binding.qsa_strerror(code) != "unknown status"
    assert binding.qsa_strerror(0) == "success"
    assert binding.qsa_strerror(99) == "unknown status"


# Fake device addresses: never dereferenced, because every call below is
# rejected (or is a no-op) before anything is enqueued.
P16 = 0x10000
P4 = 0x10004


@pytest.mark.parametrize("args,status", [
    ((P16, P16, -1, 4, 128, 10, P16), binding.QSA_ERR_SHAPE),   # nq < 0
    ((P16, P16, 1, -4, 128, 10, P16), binding.QSA_ERR_SHAPE),   # heads < 0
    ((P16, P16, 1, 4, 128, -1, P16), binding.QSA_ERR_SHAPE),    # active < 0
    ((P16, P16, 1, 4, 128, (1 << 28) + 1, P16), binding.QSA_ERR_SHAPE),  # active too large
    ((P16, P16, 1, 3, 3, 10, P16), binding.QSA_ERR_SHAPE),      # K = 9, not a multiple of 4
    ((P16, P16, 1, 2, 4097, 10, P16), binding.QSA_ERR_SHAPE),   # K > 4096
    ((P16, P16, 1, 0, 128, 10, P16), binding.QSA_ERR_SHAPE),    # K = 0
    ((None, P16, 1, 4, 128, 10, P16), binding.QSA_ERR_NULL),
    ((P16, None, 1, 4, 128, 10, P16), binding.QSA_ERR_NULL),
    ((P16, P16, 1, 4, 128, 10, None), binding.QSA_ERR_NULL),
    ((P4, P16, 1, 4, 128, 10, P16), binding.QSA_ERR_ALIGN),
    ((P16, P4, 1, 4, 128, 10, P16), binding.QSA_ERR_ALIGN),
    ((P16, P16, 1, 4, 128, 10, P16 + 2), binding.QSA_ERR_ALIGN),
    ((None, None, 0, 4, 128, 10, None), binding.QSA_OK),        # nq = 0: no-op
    ((None, None, 3, 4, 128, 0, None), binding.QSA_OK),         # no active blocks: no-op
])
def test_block_scores_argument_checks(lib, args, status):
    assert lib.qsa_block_scores(*args, None) == status


@pytest.mark.parametrize("mode,status", [(0, 0), (1, 0), (2, 0), (3, 0), (4, 6), (-1, 6)])
def test_block_scores_ex_mode_check(lib, mode, status):
    # a valid mode on an empty call is a no-op; an unknown mode is rejected first
    assert lib.qsa_block_scores_ex(None, None, 0, 4, 128, 10, None, mode, None) == status


@pytest.mark.parametrize("args,status", [
    ((P16, -1, 10, 4, P16), binding.QSA_ERR_SHAPE),
    ((P16, 1, -1, 4, P16), binding.QSA_ERR_SHAPE),
    ((P16, 1, (1 << 28) + 1, 4, P16), binding.QSA_ERR_SHAPE),   # active > QSA_MAX_ACTIVE_BLOCKS
    ((P16, 1, 10, -1, P16), binding.QSA_ERR_K),
    ((P16, 1, 10, 4097, P16), binding.QSA_ERR_K),
    ((None, 1, 10, 4, P16), binding.QSA_ERR_NULL),
    ((P16, 1, 10, 4, None), binding.QSA_ERR_NULL),
    ((P16 + 1, 1, 10, 4, P16), binding.QSA_ERR_ALIGN),
    ((P16, 1, 10, 4, P16 + 2), binding.QSA_ERR_ALIGN),
    ((None, 0, 10, 4, None), binding.QSA_OK),                   # nq = 0: no-op
    ((None, 5, 10, 0, None), binding.QSA_OK),                   # k = 0: no-op
])
def test_block_topk_argument_checks(lib, args, status):
    assert lib.qsa_block_topk(*args, None) == status


@pytest.mark.parametrize("args,status", [
    # q, kblk, nq, heads, dim, active, k, scores, ids
    ((P16, P16, -1, 4, 128, 10, 4, P16, P16), binding.QSA_ERR_SHAPE),
    ((P16, P16, 1, 3, 3, 10, 4, P16, P16), binding.QSA_ERR_SHAPE),
    ((P16, P16, 1, 4, 128, -1, 4, P16, P16), binding.QSA_ERR_SHAPE),
    ((P16, P16, 1, 4, 128, (1 << 28) + 1, 4, P16, P16), binding.QSA_ERR_SHAPE),
    ((P16, P16, 1, 4, 128, 10, -1, P16, P16), binding.QSA_ERR_K),
    ((P16, P16, 1, 4, 128, 10, 4097, P16, P16), binding.QSA_ERR_K),
    ((None, P16, 1, 4, 128, 10, 4, P16, P16), binding.QSA_ERR_NULL),
    ((P16, P16, 1, 4, 128, 10, 4, None, P16), binding.QSA_ERR_NULL),
    ((P16, P16, 1, 4, 128, 10, 4, P16, None), binding.QSA_ERR_NULL),
    ((P4, P16, 1, 4, 128, 10, 4, P16, P16), binding.QSA_ERR_ALIGN),
    ((P16, P16, 1, 4, 128, 10, 4, P16, P16 + 2), binding.QSA_ERR_ALIGN),
    ((None, None, 0, 4, 128, 10, 4, None, None), binding.QSA_OK),   # nq = 0: no-op
    ((None, None, 2, 4, 128, 0, 0, None, None), binding.QSA_OK),    # nothing to do
])
@pytest.mark.parametrize("entry", ["qsa_block_select", "qsa_block_select_noalloc"])
def test_block_select_argument_checks(lib, entry, args, status):
    assert getattr(lib, entry)(*args, None) == status


@pytest.mark.parametrize("args,status", [
    # q, kcache, vcache, ids, nq, heads, dim, k, n_cells, scale, out
    ((P16, P16, P16, P16, -1, 4, 128, 8, 100, 0.1, P16), binding.QSA_ERR_SHAPE),
    ((P16, P16, P16, P16, 1, -4, 128, 8, 100, 0.1, P16), binding.QSA_ERR_SHAPE),
    ((P16, P16, P16, P16, 1, 4, 130, 8, 100, 0.1, P16), binding.QSA_ERR_SHAPE),   # dim > 128
    ((P16, P16, P16, P16, 1, 4, 126, 8, 100, 0.1, P16), binding.QSA_ERR_SHAPE),   # dim % 4
    ((P16, P16, P16, P16, 1, 4, 0, 8, 100, 0.1, P16), binding.QSA_ERR_SHAPE),
    ((P16, P16, P16, P16, 1, 40, 128, 8, 100, 0.1, P16), binding.QSA_ERR_SHAPE),  # heads*dim > 4096
    ((P16, P16, P16, P16, 1, 4, 128, 8, -1, 0.1, P16), binding.QSA_ERR_SHAPE),    # n_cells < 0
    ((P16, P16, P16, P16, 1, 4, 128, -1, 100, 0.1, P16), binding.QSA_ERR_K),
    ((P16, P16, P16, P16, 1, 4, 128, 4097, 100, 0.1, P16), binding.QSA_ERR_K),
    ((None, P16, P16, P16, 1, 4, 128, 8, 100, 0.1, P16), binding.QSA_ERR_NULL),
    ((P16, None, P16, P16, 1, 4, 128, 8, 100, 0.1, P16), binding.QSA_ERR_NULL),
    ((P16, P16, None, P16, 1, 4, 128, 8, 100, 0.1, P16), binding.QSA_ERR_NULL),
    ((P16, P16, P16, None, 1, 4, 128, 8, 100, 0.1, P16), binding.QSA_ERR_NULL),
    ((P16, P16, P16, P16, 1, 4, 128, 8, 100, 0.1, None), binding.QSA_ERR_NULL),
    ((P4, P16, P16, P16, 1, 4, 128, 8, 100, 0.1, P16), binding.QSA_ERR_ALIGN),
    ((P16, P4, P16, P16, 1, 4, 128, 8, 100, 0.1, P16), binding.QSA_ERR_ALIGN),
    ((P16, P16, P4, P16, 1, 4, 128, 8, 100, 0.1, P16), binding.QSA_ERR_ALIGN),
    ((P16, P16, P16, P16 + 2, 1, 4, 128, 8, 100, 0.1, P16), binding.QSA_ERR_ALIGN),
    ((P16, P16, P16, P16, 1, 4, 128, 8, 100, 0.1, P16 + 2), binding.QSA_ERR_ALIGN),
    ((None, None, None, None, 0, 4, 128, 8, 100, 0.1, None), binding.QSA_OK),   # nq = 0: no-op
    ((None, None, None, None, 3, 0, 128, 8, 100, 0.1, None), binding.QSA_OK),   # heads = 0: no-op
])
def test_sparse_decode_attention_argument_checks(lib, args, status):
    assert lib.qsa_sparse_decode_attention(*args, None) == status


@pytest.mark.parametrize("args,status", [
    # q, kcode, kscale, vcode, vscale, ids, nq, heads, dim, k, n_cells, scale, out
    ((P16, P16, P16, P16, P16, P16, -1, 4, 128, 8, 100, 0.1, P16), binding.QSA_ERR_SHAPE),
    ((P16, P16, P16, P16, P16, P16, 1, 4, 120, 8, 100, 0.1, P16), binding.QSA_ERR_SHAPE),  # dim % 16
    ((P16, P16, P16, P16, P16, P16, 1, 4, 8, 8, 100, 0.1, P16), binding.QSA_ERR_SHAPE),    # dim < 16
    ((P16, P16, P16, P16, P16, P16, 1, 4, 144, 8, 100, 0.1, P16), binding.QSA_ERR_SHAPE),  # dim > 128
    ((P16, P16, P16, P16, P16, P16, 1, 40, 128, 8, 100, 0.1, P16), binding.QSA_ERR_SHAPE),
    ((P16, P16, P16, P16, P16, P16, 1, 4, 128, 8, -1, 0.1, P16), binding.QSA_ERR_SHAPE),
    ((P16, P16, P16, P16, P16, P16, 1, 4, 128, 4097, 100, 0.1, P16), binding.QSA_ERR_K),
    ((P16, P16, P16, P16, P16, P16, 1, 4, 128, -1, 100, 0.1, P16), binding.QSA_ERR_K),
    ((P16, None, P16, P16, P16, P16, 1, 4, 128, 8, 100, 0.1, P16), binding.QSA_ERR_NULL),
    ((P16, P16, None, P16, P16, P16, 1, 4, 128, 8, 100, 0.1, P16), binding.QSA_ERR_NULL),
    ((P16, P16, P16, None, P16, P16, 1, 4, 128, 8, 100, 0.1, P16), binding.QSA_ERR_NULL),
    ((P16, P16, P16, P16, None, P16, 1, 4, 128, 8, 100, 0.1, P16), binding.QSA_ERR_NULL),
    ((P16, P16, P16, P16, P16, None, 1, 4, 128, 8, 100, 0.1, P16), binding.QSA_ERR_NULL),
    ((P16, P16, P16, P16, P16, P16, 1, 4, 128, 8, 100, 0.1, None), binding.QSA_ERR_NULL),
    ((P16, P16 + 8, P16, P16, P16, P16, 1, 4, 128, 8, 100, 0.1, P16), binding.QSA_ERR_ALIGN),
    ((P16, P16, P16 + 1, P16, P16, P16, 1, 4, 128, 8, 100, 0.1, P16), binding.QSA_ERR_ALIGN),
    ((P16, P16, P16, P16, P16 + 1, P16, 1, 4, 128, 8, 100, 0.1, P16), binding.QSA_ERR_ALIGN),
    ((P16 + 4, P16, P16, P16, P16, P16, 1, 4, 128, 8, 100, 0.1, P16), binding.QSA_ERR_ALIGN),
    ((None, None, None, None, None, None, 0, 4, 128, 8, 100, 0.1, None), binding.QSA_OK),
])
def test_sparse_decode_attention_i8_argument_checks(lib, args, status):
    assert lib.qsa_sparse_decode_attention_i8(*args, None) == status


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 4, 64)
    with pytest.raises(ValueError):
        binding.qsa_block_scores(q, q)
    with pytest.raises(ValueError):
        binding.qsa_block_topk(torch.zeros(1, 8), 2)
