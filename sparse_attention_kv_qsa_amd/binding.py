"""ctypes binding of libqsa.so (C ABI in include/qsa.h).

Argument marshalling only: tensors are checked for dtype, device, layout and
shape, outputs are allocated with torch when the caller passes none, and the
work is enqueued on the tensor device's current torch stream.  Every step of
the computation runs in the library's HIP kernels.  There is no fallback: a
missing library, or tensors that are not on a GPU, raise.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libqsa.so"

# Mirrors of include/qsa.h.
QSA_OK, QSA_ERR_NULL, QSA_ERR_SHAPE, QSA_ERR_K, QSA_ERR_ALIGN, QSA_ERR_LAUNCH = 0, 1, 2, 3, 4, 5
QSA_ERR_MODE = 6
QSA_ERR_NOMEM = 7
QSA_ERR_SCRATCH = 8
QSA_NOALLOC_SCRATCH_BYTES = 2097152
QSA_MAX_HEAD_DIM = 4096
TOPK_MAX_K = 4096
MAX_ACTIVE_BLOCKS = 1 << 28
TOPK_FEW_ROWS = 16
QSA_SCORES_AUTO, QSA_SCORES_FP32, QSA_SCORES_BF16X3, QSA_SCORES_F16X2 = 0, 1, 2, 3
QSA_ATTN_MAX_DIM = 128
SCORE_MODES = {"auto": QSA_SCORES_AUTO, "fp32": QSA_SCORES_FP32, "bf16x3": QSA_SCORES_BF16X3,
               "f16x2": QSA_SCORES_F16X2}

# Entry points declared in include/qsa.h: name -> (restype, argtypes).
_VP, _I = ctypes.c_void_p, ctypes.c_int
SIGNATURES = {
    "qsa_block_scores": (_I, [_VP, _VP, _I, _I, _I, _I, _VP, _VP]),
    "qsa_block_scores_ex": (_I, [_VP, _VP, _I, _I, _I, _I, _VP, _I, _VP]),
    "qsa_block_topk": (_I, [_VP, _I, _I, _I, _VP, _VP]),
    "qsa_block_select": (_I, [_VP, _VP, _I, _I, _I, _I, _I, _VP, _VP, _VP]),
    "qsa_block_select_noalloc": (_I, [_VP, _VP, _I, _I, _I, _I, _I, _VP, _VP, _VP]),
    "qsa_sparse_decode_attention": (_I, [_VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, ctypes.c_float,
                                         _VP, _VP]),
    "qsa_sparse_decode_attention_i8": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _I,
                                            ctypes.c_float, _VP, _VP]),
    "qsa_strerror": (ctypes.c_char_p, [_I]),
}

_lib = None


class QSAError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status} ({qsa_strerror(status)})")


def library_path() -> str:
    return os.environ.get("QSA_LIBRARY", os.path.join(_HERE, _LIB_NAME))


def load_library():
    """Load libqsa.so once and attach the C signatures; raises if it is not built."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with "
                               "`python -m sparse_attention_kv_qsa_amd.build` (hipcc, gfx950)")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def qsa_strerror(status: int) -> str:
    return load_library().qsa_strerror(int(status)).decode()


# The current stream's raw handle without building a torch.cuda.Stream object
# (the public route below costs about 2 us per call).
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_handle(device: torch.device):
    if _raw_stream is not None:
        return _raw_stream(device.index) or None
    return torch.cuda.current_stream(device).cuda_stream or None


def _launch(device: torch.device, fn, *args):
    """fn(*args, stream) with `device` current: the library allocates its
    scratch on the current device.  The device switch is skipped when it is
    already current (the common case, about 1 us saved per call)."""
    if device.index == torch.cuda.current_device():
        return fn(*args, _stream_handle(device))
    with torch.cuda.device(device):
        return fn(*args, _stream_handle(device))


def _require_gpu_f32(name: str, t: torch.Tensor, ndim: int):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != torch.float32:
        raise ValueError(f"{name} must be float32, got {t.dtype}")
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {ndim}-d tensor")


def qsa_block_scores_ex(q: torch.Tensor, kblk: torch.Tensor, active_blocks: int | None = None,
                        scores: torch.Tensor | None = None, mode="auto") -> torch.Tensor:
    """Scores [nq, active_blocks] of q [nq, heads, dim] against kblk [C, heads, dim].

    Only rows [0, active_blocks) of kblk are read (default: all C rows).
    mode: "auto" | "fp32" | "bf16x3" | "f16x2" (or the QSA_SCORES_* integer).
    """
    _require_gpu_f32("q", q, 3)
    _require_gpu_f32("kblk", kblk, 3)
    nq, heads, dim = q.shape
    if kblk.shape[1:] != q.shape[1:] or kblk.device != q.device:
        raise ValueError("kblk must be [capacity, heads, dim] on q's device")
    a = kblk.shape[0] if active_blocks is None else int(active_blocks)
    if not 0 <= a <= kblk.shape[0]:
        raise ValueError(f"active_blocks={a} outside [0, {kblk.shape[0]}]")
    m = SCORE_MODES[mode] if isinstance(mode, str) else int(mode)
    if scores is None:
        scores = torch.empty((nq, a), dtype=torch.float32, device=q.device)
    else:
        _require_gpu_f32("scores", scores, 2)
        if tuple(scores.shape) != (nq, a) or scores.device != q.device:
            raise ValueError(f"scores must be [{nq}, {a}] on q's device")
    st = _launch(q.device, load_library().qsa_block_scores_ex, q.data_ptr(), kblk.data_ptr(), nq,
                 heads, dim, a, scores.data_ptr(), m)
    if st != QSA_OK:
        raise QSAError(st, "qsa_block_scores_ex")
    return scores


def qsa_block_scores(q: torch.Tensor, kblk: torch.Tensor, active_blocks: int | None = None,
                     scores: torch.Tensor | None = None) -> torch.Tensor:
    """Scores [nq, active_blocks] with the library's default precision mode."""
    return qsa_block_scores_ex(q, kblk, active_blocks, scores, QSA_SCORES_AUTO)


def qsa_block_select(q: torch.Tensor, kblk: torch.Tensor, k: int, active_blocks: int | None = None,
                     scores: torch.Tensor | None = None, ids: torch.Tensor | None = None):
    """(scores [nq, active_blocks], ids [nq, k]) in one call: the scores of
    qsa_block_scores and the top-k of qsa_block_topk on them."""
    return _select("qsa_block_select", q, kblk, k, active_blocks, scores, ids)


def qsa_block_select_noalloc(q: torch.Tensor, kblk: torch.Tensor, k: int,
                             active_blocks: int | None = None, scores: torch.Tensor | None = None,
                             ids: torch.Tensor | None = None):
    """qsa_block_select with the library's scratch in a static device array
    instead of an allocation (the library calls no hipMalloc; outputs the
    caller does not pass are still allocated here, by torch).  Calls that
    overlap on one GPU race."""
    return _select("qsa_block_select_noalloc", q, kblk, k, active_blocks, scores, ids)


def _select(name, q, kblk, k, active_blocks, scores, ids):
    _require_gpu_f32("q", q, 3)
    _require_gpu_f32("kblk", kblk, 3)
    nq, heads, dim = q.shape
    if kblk.shape[1:] != (heads, dim) or kblk.device != q.device:
        raise ValueError("kblk must be [C, heads, dim] on q's device")
    a = kblk.shape[0] if active_blocks is None else int(active_blocks)
    if not 0 <= a <= kblk.shape[0]:
        raise ValueError(f"active_blocks={a} outside [0, {kblk.shape[0]}]")
    k = int(k)
    if scores is None:
        scores = torch.empty((nq, a), dtype=torch.float32, device=q.device)
    elif tuple(scores.shape) != (nq, a) or scores.device != q.device or \
            scores.dtype != torch.float32 or not scores.is_contiguous():
        raise ValueError(f"scores must be a contiguous float32 [{nq}, {a}] tensor on q's device")
    if ids is None:
        ids = torch.empty((nq, max(k, 0)), dtype=torch.int32, device=q.device)
    elif tuple(ids.shape) != (nq, k) or ids.device != q.device or ids.dtype != torch.int32 or \
            not ids.is_contiguous():
        raise ValueError(f"ids must be a contiguous int32 [{nq}, {k}] tensor on q's device")
    st = _launch(q.device, getattr(load_library(), name), q.data_ptr(), kblk.data_ptr(), nq,
                 heads, dim, a, k, scores.data_ptr(), ids.data_ptr())
    if st != QSA_OK:
        raise QSAError(st, name)
    return scores, ids


def qsa_block_topk(scores: torch.Tensor, k: int, ids: torch.Tensor | None = None) -> torch.Tensor:
    """Rank-ordered top-k block ids [nq, k] (int32, -1 padded) of scores [nq, active_blocks]."""
    _require_gpu_f32("scores", scores, 2)
    nq, a = scores.shape
    k = int(k)
    if ids is None:
        ids = torch.empty((nq, max(k, 0)), dtype=torch.int32, device=scores.device)
    elif (ids.dtype != torch.int32 or tuple(ids.shape) != (nq, k) or not ids.is_contiguous()
          or ids.device != scores.device):
        raise ValueError(f"ids must be a contiguous int32 [{nq}, {k}] tensor on scores' device")
    st = _launch(scores.device, load_library().qsa_block_topk, scores.data_ptr() if a else None,
                 nq, a, k, ids.data_ptr() if ids.numel() else None)
    if st != QSA_OK:
        raise QSAError(st, "qsa_block_topk")
    return ids


def qsa_sparse_decode_attention(q: torch.Tensor, kcache: torch.Tensor, vcache: torch.Tensor,
                                ids: torch.Tensor, n_cells: int | None = None,
                                scale: float | None = None,
                                out: torch.Tensor | None = None) -> torch.Tensor:
    """Attention out [nq, heads, dim] of q [nq, heads, dim] over the cells of the
    blocks ids [nq, k] (int32, -1 skipped) in kcache/vcache [cells, heads, dim];
    cells at or past n_cells (default: all rows) are skipped; scale defaults to
    1/sqrt(dim)."""
    _require_gpu_f32("q", q, 3)
    _require_gpu_f32("kcache", kcache, 3)
    _require_gpu_f32("vcache", vcache, 3)
    nq, heads, dim = q.shape
    if kcache.shape[1:] != (heads, dim) or tuple(vcache.shape) != tuple(kcache.shape) or \
            kcache.device != q.device or vcache.device != q.device:
        raise ValueError("kcache and vcache must be [cells, heads, dim] on q's device")
    n = kcache.shape[0] if n_cells is None else int(n_cells)
    if not 0 <= n <= kcache.shape[0]:
        raise ValueError(f"n_cells={n} outside [0, {kcache.shape[0]}]")
    if ids.dtype != torch.int32 or ids.dim() != 2 or ids.shape[0] != nq or \
            not ids.is_contiguous() or ids.device != q.device:
        raise ValueError(f"ids must be a contiguous int32 [{nq}, k] tensor on q's device")
    k = ids.shape[1]
    sc = 1.0 / float(dim) ** 0.5 if scale is None else float(scale)
    if out is None:
        out = torch.empty((nq, heads, dim), dtype=torch.float32, device=q.device)
    elif tuple(out.shape) != (nq, heads, dim) or out.dtype != torch.float32 or \
            not out.is_contiguous() or out.device != q.device:
        raise ValueError(f"out must be a contiguous float32 [{nq}, {heads}, {dim}] tensor on q's device")
    st = _launch(q.device, load_library().qsa_sparse_decode_attention, q.data_ptr(),
                 kcache.data_ptr(), vcache.data_ptr(), ids.data_ptr() if ids.numel() else None,
                 nq, heads, dim, k, n, sc, out.data_ptr())
    if st != QSA_OK:
        raise QSAError(st, "qsa_sparse_decode_attention")
    return out


def qsa_sparse_decode_attention_i8(q: torch.Tensor, kcode: torch.Tensor, kscale: torch.Tensor,
                                   vcode: torch.Tensor, vscale: torch.Tensor, ids: torch.Tensor,
                                   n_cells: int | None = None, scale: float | None = None,
                                   out: torch.Tensor | None = None) -> torch.Tensor:
    """qsa_sparse_decode_attention over an int8 pool: kcode/vcode [cells, heads,
    dim] int8 codes, kscale/vscale [cells, heads] binary16 scales (float16, or
    int16 bit patterns); an element stands for code * scale."""
    _require_gpu_f32("q", q, 3)
    nq, heads, dim = q.shape
    for name, t in (("kcode", kcode), ("vcode", vcode)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.int8 or t.dim() != 3 or \
                not t.is_contiguous() or t.device != q.device or t.shape[1:] != (heads, dim):
            raise ValueError(f"{name} must be a contiguous int8 [cells, {heads}, {dim}] tensor "
                             "on q's device")
    cells = kcode.shape[0]
    if vcode.shape[0] != cells:
        raise ValueError("kcode and vcode must have the same number of cells")
    for name, t in (("kscale", kscale), ("vscale", vscale)):
        if not isinstance(t, torch.Tensor) or t.dtype not in (torch.float16, torch.int16) or \
                tuple(t.shape) != (cells, heads) or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous float16 (or int16 bits) "
                             f"[{cells}, {heads}] tensor on q's device")
    n = cells if n_cells is None else int(n_cells)
    if not 0 <= n <= cells:
        raise ValueError(f"n_cells={n} outside [0, {cells}]")
    if ids.dtype != torch.int32 or ids.dim() != 2 or ids.shape[0] != nq or \
            not ids.is_contiguous() or ids.device != q.device:
        raise ValueError(f"ids must be a contiguous int32 [{nq}, k] tensor on q's device")
    k = ids.shape[1]
    sc = 1.0 / float(dim) ** 0.5 if scale is None else float(scale)
    if out is None:
        out = torch.empty((nq, heads, dim), dtype=torch.float32, device=q.device)
    elif tuple(out.shape) != (nq, heads, dim) or out.dtype != torch.float32 or \
            not out.is_contiguous() or out.device != q.device:
        raise ValueError(f"out must be a contiguous float32 [{nq}, {heads}, {dim}] tensor on q's device")
    st = _launch(q.device, load_library().qsa_sparse_decode_attention_i8, q.data_ptr(),
                 kcode.data_ptr(), kscale.data_ptr(), vcode.data_ptr(), vscale.data_ptr(),
                 ids.data_ptr() if ids.numel() else None, nq, heads, dim, k, n, sc,
                 out.data_ptr())
    if st != QSA_OK:
        raise QSAError(st, "qsa_sparse_decode_attention_i8")
    return out


# Short aliases.
block_scores = qsa_block_scores
block_topk = qsa_block_topk
sparse_decode_attention = qsa_sparse_decode_attention
sparse_decode_attention_i8 = qsa_sparse_decode_attention_i8
