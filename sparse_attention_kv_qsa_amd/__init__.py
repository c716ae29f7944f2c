"""QSA block selection on MI355X (gfx950): exact block scoring + radix top-k.

The compute lives in ``libqsa.so`` (hand-written HIP for CDNA4, C ABI declared
in ``include/qsa.h``).  ``qsa_block_scores`` / ``qsa_block_topk`` /
``qsa_block_select`` (and ``qsa_block_select_noalloc``, whose scratch is a
static device array) / ``qsa_sparse_decode_attention`` (and ``_i8``, over an
int8 key/value pool) here are thin ctypes
bindings with the same names as the C entry points: they marshal torch
tensors and the current HIP stream, nothing more.  There is no CPU fallback:
calling them without the built library, or with tensors that are not on the
GPU, raises.
"""
from .synth import (WORKLOADS, HEADLINE, Workload, make_batch, make_random, make_kv,  # noqa: F401
                    make_pool_i8, fingerprint)


def __getattr__(name):
    # The binding loads libqsa.so (and torch) on first use only, so the
    # generator can be imported on hosts without the library.
    if name in ("qsa_block_scores", "qsa_block_scores_ex", "qsa_block_topk", "qsa_block_select",
                "qsa_block_select_noalloc",
                "qsa_sparse_decode_attention", "sparse_decode_attention", "QSA_ATTN_MAX_DIM",
                "qsa_sparse_decode_attention_i8", "sparse_decode_attention_i8",
                "qsa_strerror", "TOPK_FEW_ROWS",
                "QSAError", "SCORE_MODES",
                "load_library", "library_path", "TOPK_MAX_K", "block_scores", "block_topk"):
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
