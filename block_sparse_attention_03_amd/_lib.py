"""ctypes binding of libmsa.so (include/msa.h).

Argument marshalling only: every function checks the tensors it is given
(device, dtype, contiguity, shape), packs ``msa_dims_t`` and calls the C entry
point of the same name on the current HIP stream; ``prepare_<name>`` does the
checking and packing once and returns a PreparedCall that repeats the call.
All arithmetic runs in the library's HIP kernels; there is no CPU fallback,
and loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmsa.so")

MSA_SUCCESS = 0
MSA_ERROR_INVALID_VALUE = 1
MSA_ERROR_NOT_SUPPORTED = 2
MSA_ERROR_WORKSPACE = 3
MSA_ERROR_LAUNCH = 4

EXPORTED = (
    "msa_index_score", "msa_topk_blocks", "msa_build_page_table", "msa_sparse_attn_decode",
    "msa_sparse_attn_prefill", "msa_decode_workspace_size", "msa_prefill_workspace_size",
    "msa_status_string", "msa_abi_version", "msa_decode_step", "msa_decode_step_workspace_size",
    "msa_dense_attn_decode", "msa_dense_decode_workspace_size", "msa_dense_attn_prefill",
    "msa_validate_inputs", "msa_append_kv", "msa_decode_step_append", "msa_decode_step_noalloc",
    "msa_multi_query_step", "msa_multi_query_step_workspace_size",
)

MSA_STATIC_SCRATCH_BYTES = 32 << 20  # include/msa.h


class msa_dims_t(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("num_idx_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("idx_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
    ]


class MsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} ({status})")
        self.status = status


_lib = None


def lib():
    """The loaded libmsa.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python block_sparse_attention_03_amd/build.py`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        D = ctypes.POINTER(msa_dims_t)
        L.msa_index_score.argtypes = [D, I32, P, P, P, P, P, P, P]
        L.msa_topk_blocks.argtypes = [D, I32, P, P, P, P, P]
        L.msa_build_page_table.argtypes = [D, P, P, P, P, P, P]
        L.msa_sparse_attn_decode.argtypes = [D, P, P, P, P, P, P, P, P, SZ, P]
        L.msa_sparse_attn_prefill.argtypes = [D, I32, P, P, P, P, P, P, P, P, P, P, SZ, P]
        L.msa_decode_step.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
        L.msa_decode_step_append.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
        L.msa_decode_step_noalloc.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P]
        L.msa_decode_step_workspace_size.argtypes = [D]
        L.msa_decode_step_workspace_size.restype = SZ
        L.msa_multi_query_step.argtypes = [D, I32, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
        L.msa_multi_query_step_workspace_size.argtypes = [D, I32]
        L.msa_multi_query_step_workspace_size.restype = SZ
        L.msa_dense_attn_decode.argtypes = [D, P, P, P, P, P, P, P, P, SZ, P]
        L.msa_dense_attn_prefill.argtypes = [D, I32, P, P, P, P, P, P, P, P, P]
        L.msa_validate_inputs.argtypes = [D, I32, P, P, P, P, P]
        L.msa_append_kv.argtypes = [D, I32, P, P, P, P, P, P, P, P, P, P]
        L.msa_dense_decode_workspace_size.argtypes = [D]
        L.msa_dense_decode_workspace_size.restype = SZ
        for f in ("msa_index_score", "msa_topk_blocks", "msa_build_page_table",
                  "msa_sparse_attn_decode", "msa_sparse_attn_prefill", "msa_decode_step",
                  "msa_dense_attn_decode", "msa_dense_attn_prefill", "msa_validate_inputs",
                  "msa_append_kv", "msa_decode_step_append", "msa_decode_step_noalloc",
                  "msa_multi_query_step"):
            getattr(L, f).restype = ctypes.c_int
        L.msa_decode_workspace_size.argtypes = [D]
        L.msa_decode_workspace_size.restype = SZ
        L.msa_prefill_workspace_size.argtypes = [D, I32]
        L.msa_prefill_workspace_size.restype = SZ
        L.msa_status_string.argtypes = [ctypes.c_int]
        L.msa_status_string.restype = ctypes.c_char_p
        L.msa_abi_version.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().msa_status_string(int(status)).decode()


def abi_version() -> int:
    return int(lib().msa_abi_version())


def make_dims(num_seqs, num_q_heads, num_kv_heads, max_blocks_per_seq, num_pages,
              num_idx_heads=1, head_dim=128, idx_dim=64, block_size=128, topk=16,
              softmax_scale=0.0) -> msa_dims_t:
    return msa_dims_t(num_seqs, num_q_heads, num_kv_heads, num_idx_heads, head_dim, idx_dim,
                      block_size, topk, max_blocks_per_seq, num_pages, softmax_scale)


def dims_for(cfg) -> msa_dims_t:
    """msa_dims_t of an inputs.MsaConfig."""
    return make_dims(cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads, cfg.max_blocks,
                     cfg.num_pages, cfg.num_idx_heads, cfg.head_dim, cfg.idx_dim,
                     cfg.block_size, cfg.topk)


def _ptr(t: Optional[torch.Tensor], dtype, name: str, shape=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a device tensor (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(status: int, where: str):
    if status != MSA_SUCCESS:
        raise MsaError(status, where)


BF16, I32, F32 = torch.bfloat16, torch.int32, torch.float32


class PreparedCall:
    """One entry point with its tensors checked and its arguments packed once.
    Calling it passes the same pointers again on the current (or a given) HIP
    stream: for loops that reuse their buffers (decode layers, benchmarks),
    where checking every tensor on every call would cost more host time than
    the kernels take on the GPU.  The tensors are referenced here, so their
    storage stays allocated; their contents may change between calls."""
    __slots__ = ("_fn", "_args", "_where", "_keep")

    def __init__(self, fn, args, where, keep):
        self._fn, self._args, self._where, self._keep = fn, args, where, keep

    def __call__(self, stream=None):
        _check(self._fn(*self._args, _stream(stream)), self._where)


def prepare_msa_index_score(dims, total_q, q_idx, kidx_cache, block_table, seq_lens, cu_q, scores):
    """msa_index_score with its arguments checked and packed once: returns a
    PreparedCall that repeats the call, on the current (or a given) stream."""
    d = dims
    H, B, W = d.num_kv_heads, d.num_seqs, d.max_blocks_per_seq
    args = (_ptr(q_idx, BF16, "q_idx", (total_q, H, d.idx_dim)),
            _ptr(kidx_cache, BF16, "kidx_cache", (d.num_pages, d.num_idx_heads, d.block_size, d.idx_dim)),
            _ptr(block_table, I32, "block_table", (B, W)), _ptr(seq_lens, I32, "seq_lens", (B,)),
            _ptr(cu_q, I32, "cu_q", (B + 1,)), _ptr(scores, F32, "scores", (total_q, H, W)))
    return PreparedCall(lib().msa_index_score, (ctypes.byref(d), total_q, *args), "msa_index_score",
                        (d, q_idx, kidx_cache, block_table, seq_lens, cu_q, scores))


def msa_index_score(dims, total_q, q_idx, kidx_cache, block_table, seq_lens, cu_q, scores,
                    stream=None):
    prepare_msa_index_score(dims, total_q, q_idx, kidx_cache, block_table, seq_lens, cu_q,
                            scores)(stream)


def prepare_msa_topk_blocks(dims, total_q, scores, seq_lens, cu_q, sel):
    """msa_topk_blocks with its arguments checked and packed once: returns a
    PreparedCall that repeats the call, on the current (or a given) stream."""
    d = dims
    H, B = d.num_kv_heads, d.num_seqs
    args = (_ptr(scores, F32, "scores", (total_q, H, d.max_blocks_per_seq)),
            _ptr(seq_lens, I32, "seq_lens", (B,)), _ptr(cu_q, I32, "cu_q", (B + 1,)),
            _ptr(sel, I32, "sel", (total_q, H, d.topk)))
    return PreparedCall(lib().msa_topk_blocks, (ctypes.byref(d), total_q, *args), "msa_topk_blocks",
                        (d, scores, seq_lens, cu_q, sel))


def msa_topk_blocks(dims, total_q, scores, seq_lens, cu_q, sel, stream=None):
    prepare_msa_topk_blocks(dims, total_q, scores, seq_lens, cu_q, sel)(stream)


def prepare_msa_build_page_table(dims, sel, block_table, seq_lens, page_table, row_lens):
    """msa_build_page_table with its arguments checked and packed once: returns a
    PreparedCall that repeats the call, on the current (or a given) stream."""
    d = dims
    B, H = d.num_seqs, d.num_kv_heads
    args = (_ptr(sel, I32, "sel", (B, H, d.topk)),
            _ptr(block_table, I32, "block_table", (B, d.max_blocks_per_seq)),
            _ptr(seq_lens, I32, "seq_lens", (B,)),
            _ptr(page_table, I32, "page_table", (B * H, d.topk)),
            _ptr(row_lens, I32, "row_lens", (B * H,)))
    return PreparedCall(lib().msa_build_page_table, (ctypes.byref(d), *args),
                        "msa_build_page_table",
                        (d, sel, block_table, seq_lens, page_table, row_lens))


def msa_build_page_table(dims, sel, block_table, seq_lens, page_table, row_lens, stream=None):
    prepare_msa_build_page_table(dims, sel, block_table, seq_lens, page_table, row_lens)(stream)


def msa_decode_workspace_size(dims) -> int:
    return int(lib().msa_decode_workspace_size(ctypes.byref(dims)))


def msa_prefill_workspace_size(dims, total_q) -> int:
    return int(lib().msa_prefill_workspace_size(ctypes.byref(dims), total_q))


def prepare_msa_sparse_attn_decode(dims, q, k_cache, v_cache, page_table, row_lens, out, lse,
                                   workspace):
    """msa_sparse_attn_decode with its arguments checked and packed once: returns a
    PreparedCall that repeats the call, on the current (or a given) stream."""
    d = dims
    B, Hq, H = d.num_seqs, d.num_q_heads, d.num_kv_heads
    cache = (d.num_pages, H, d.block_size, d.head_dim)
    args = (_ptr(q, BF16, "q", (B, Hq, d.head_dim)), _ptr(k_cache, BF16, "k_cache", cache),
            _ptr(v_cache, BF16, "v_cache", cache),
            _ptr(page_table, I32, "page_table", (B * H, d.topk)),
            _ptr(row_lens, I32, "row_lens", (B * H,)),
            _ptr(out, BF16, "out", (B, Hq, d.head_dim)),
            _ptr(lse, F32, "lse", (B, Hq)) if lse is not None else None,
            _ptr(workspace, torch.uint8, "workspace"))
    nbytes = workspace.numel() if workspace is not None else 0
    return PreparedCall(lib().msa_sparse_attn_decode, (ctypes.byref(d), *args, nbytes),
                        "msa_sparse_attn_decode",
                        (d, q, k_cache, v_cache, page_table, row_lens, out, lse, workspace))


def msa_sparse_attn_decode(dims, q, k_cache, v_cache, page_table, row_lens, out, lse, workspace,
                           stream=None):
    prepare_msa_sparse_attn_decode(dims, q, k_cache, v_cache, page_table, row_lens, out, lse,
                                   workspace)(stream)


def prepare_msa_sparse_attn_prefill(dims, total_q, q, k_cache, v_cache, block_table, seq_lens, cu_q,
                                    sel, out, lse, workspace):
    """msa_sparse_attn_prefill with its arguments checked and packed once: returns a
    PreparedCall that repeats the call, on the current (or a given) stream."""
    d = dims
    B, Hq, H = d.num_seqs, d.num_q_heads, d.num_kv_heads
    cache = (d.num_pages, H, d.block_size, d.head_dim)
    args = (_ptr(q, BF16, "q", (total_q, Hq, d.head_dim)), _ptr(k_cache, BF16, "k_cache", cache),
            _ptr(v_cache, BF16, "v_cache", cache),
            _ptr(block_table, I32, "block_table", (B, d.max_blocks_per_seq)),
            _ptr(seq_lens, I32, "seq_lens", (B,)), _ptr(cu_q, I32, "cu_q", (B + 1,)),
            _ptr(sel, I32, "sel", (total_q, H, d.topk)),
            _ptr(out, BF16, "out", (total_q, Hq, d.head_dim)),
            _ptr(lse, F32, "lse", (total_q, Hq)) if lse is not None else None,
            _ptr(workspace, torch.uint8, "workspace"))
    nbytes = workspace.numel() if workspace is not None else 0
    return PreparedCall(lib().msa_sparse_attn_prefill, (ctypes.byref(d), total_q, *args, nbytes),
                        "msa_sparse_attn_prefill",
                        (d, q, k_cache, v_cache, block_table, seq_lens, cu_q, sel, out, lse,
                         workspace))


def msa_sparse_attn_prefill(dims, total_q, q, k_cache, v_cache, block_table, seq_lens, cu_q, sel,
                            out, lse, workspace, stream=None):
    prepare_msa_sparse_attn_prefill(dims, total_q, q, k_cache, v_cache, block_table, seq_lens, cu_q,
                                    sel, out, lse, workspace)(stream)


def msa_decode_step_workspace_size(dims) -> int:
    return int(lib().msa_decode_step_workspace_size(ctypes.byref(dims)))


def prepare_msa_decode_step(dims, q_idx, kidx_cache, q, k_cache, v_cache, block_table, seq_lens,
                            out, lse, sel, workspace):
    """msa_decode_step with its arguments checked and packed once: returns a
    PreparedCall that repeats the call, on the current (or a given) stream."""
    d = dims
    B, Hq, H = d.num_seqs, d.num_q_heads, d.num_kv_heads
    cache = (d.num_pages, H, d.block_size, d.head_dim)
    args = (_ptr(q_idx, BF16, "q_idx", (B, H, d.idx_dim)),
            _ptr(kidx_cache, BF16, "kidx_cache", (d.num_pages, d.num_idx_heads, d.block_size, d.idx_dim)),
            _ptr(q, BF16, "q", (B, Hq, d.head_dim)), _ptr(k_cache, BF16, "k_cache", cache),
            _ptr(v_cache, BF16, "v_cache", cache),
            _ptr(block_table, I32, "block_table", (B, d.max_blocks_per_seq)),
            _ptr(seq_lens, I32, "seq_lens", (B,)),
            _ptr(out, BF16, "out", (B, Hq, d.head_dim)),
            _ptr(lse, F32, "lse", (B, Hq)) if lse is not None else None,
            _ptr(sel, I32, "sel", (B, H, d.topk)) if sel is not None else None,
            _ptr(workspace, torch.uint8, "workspace"))
    nbytes = workspace.numel() if workspace is not None else 0
    return PreparedCall(lib().msa_decode_step, (ctypes.byref(d), *args, nbytes), "msa_decode_step",
                        (d, q_idx, kidx_cache, q, k_cache, v_cache, block_table, seq_lens, out,
                         lse, sel, workspace))


def msa_decode_step(dims, q_idx, kidx_cache, q, k_cache, v_cache, block_table, seq_lens, out, lse,
                    sel, workspace, stream=None):
    prepare_msa_decode_step(dims, q_idx, kidx_cache, q, k_cache, v_cache, block_table, seq_lens,
                            out, lse, sel, workspace)(stream)


def msa_multi_query_step_workspace_size(dims, total_q: int) -> int:
    return int(lib().msa_multi_query_step_workspace_size(ctypes.byref(dims), total_q))


def prepare_msa_multi_query_step(dims, total_q, q_idx, kidx_cache, q, k_cache, v_cache,
                                 block_table, seq_lens, cu_q, out, lse, sel, workspace):
    """msa_multi_query_step with its arguments checked and packed once: returns
    a PreparedCall that repeats the call, on the current (or a given) stream."""
    d = dims
    B, Hq, H, T = d.num_seqs, d.num_q_heads, d.num_kv_heads, total_q
    cache = (d.num_pages, H, d.block_size, d.head_dim)
    args = (_ptr(q_idx, BF16, "q_idx", (T, H, d.idx_dim)),
            _ptr(kidx_cache, BF16, "kidx_cache", (d.num_pages, d.num_idx_heads, d.block_size, d.idx_dim)),
            _ptr(q, BF16, "q", (T, Hq, d.head_dim)), _ptr(k_cache, BF16, "k_cache", cache),
            _ptr(v_cache, BF16, "v_cache", cache),
            _ptr(block_table, I32, "block_table", (B, d.max_blocks_per_seq)),
            _ptr(seq_lens, I32, "seq_lens", (B,)), _ptr(cu_q, I32, "cu_q", (B + 1,)),
            _ptr(out, BF16, "out", (T, Hq, d.head_dim)),
            _ptr(lse, F32, "lse", (T, Hq)) if lse is not None else None,
            _ptr(sel, I32, "sel", (T, H, d.topk)) if sel is not None else None,
            _ptr(workspace, torch.uint8, "workspace"))
    nbytes = workspace.numel() if workspace is not None else 0
    return PreparedCall(lib().msa_multi_query_step, (ctypes.byref(d), T, *args, nbytes),
                        "msa_multi_query_step",
                        (d, q_idx, kidx_cache, q, k_cache, v_cache, block_table, seq_lens, cu_q,
                         out, lse, sel, workspace))


def msa_multi_query_step(dims, total_q, q_idx, kidx_cache, q, k_cache, v_cache, block_table,
                         seq_lens, cu_q, out, lse, sel, workspace, stream=None):
    prepare_msa_multi_query_step(dims, total_q, q_idx, kidx_cache, q, k_cache, v_cache,
                                 block_table, seq_lens, cu_q, out, lse, sel, workspace)(stream)


def prepare_msa_decode_step_noalloc(dims, q_idx, kidx_cache, q, k_cache, v_cache, block_table,
                                    seq_lens, out, lse, sel):
    """msa_decode_step_noalloc (the decode step in the library's own static
    scratch, no workspace) with its arguments checked and packed once: returns
    a PreparedCall that repeats the call, on the current (or a given) stream."""
    d = dims
    B, Hq, H = d.num_seqs, d.num_q_heads, d.num_kv_heads
    cache = (d.num_pages, H, d.block_size, d.head_dim)
    args = (_ptr(q_idx, BF16, "q_idx", (B, H, d.idx_dim)),
            _ptr(kidx_cache, BF16, "kidx_cache", (d.num_pages, d.num_idx_heads, d.block_size, d.idx_dim)),
            _ptr(q, BF16, "q", (B, Hq, d.head_dim)), _ptr(k_cache, BF16, "k_cache", cache),
            _ptr(v_cache, BF16, "v_cache", cache),
            _ptr(block_table, I32, "block_table", (B, d.max_blocks_per_seq)),
            _ptr(seq_lens, I32, "seq_lens", (B,)),
            _ptr(out, BF16, "out", (B, Hq, d.head_dim)),
            _ptr(lse, F32, "lse", (B, Hq)) if lse is not None else None,
            _ptr(sel, I32, "sel", (B, H, d.topk)) if sel is not None else None)
    return PreparedCall(lib().msa_decode_step_noalloc, (ctypes.byref(d), *args),
                        "msa_decode_step_noalloc",
                        (d, q_idx, kidx_cache, q, k_cache, v_cache, block_table, seq_lens, out,
                         lse, sel))


def msa_decode_step_noalloc(dims, q_idx, kidx_cache, q, k_cache, v_cache, block_table, seq_lens,
                            out, lse, sel, stream=None):
    """msa_decode_step without a workspace: the library's static per-GPU scratch
    (MSA_STATIC_SCRATCH_BYTES) holds the step's partials; nothing is allocated."""
    prepare_msa_decode_step_noalloc(dims, q_idx, kidx_cache, q, k_cache, v_cache, block_table,
                                    seq_lens, out, lse, sel)(stream)


def prepare_msa_decode_step_append(dims, k_new, v_new, kidx_new, q_idx, kidx_cache, q, k_cache,
                                   v_cache, block_table, seq_lens, out, lse, sel, workspace):
    """msa_decode_step_append with its arguments checked and packed once: returns
    a PreparedCall that repeats the call, on the current (or a given) stream."""
    d = dims
    B, Hq, H = d.num_seqs, d.num_q_heads, d.num_kv_heads
    cache = (d.num_pages, H, d.block_size, d.head_dim)
    args = (_ptr(k_new, BF16, "k_new", (B, H, d.head_dim)),
            _ptr(v_new, BF16, "v_new", (B, H, d.head_dim)),
            _ptr(kidx_new, BF16, "kidx_new", (B, d.num_idx_heads, d.idx_dim)),
            _ptr(q_idx, BF16, "q_idx", (B, H, d.idx_dim)),
            _ptr(kidx_cache, BF16, "kidx_cache", (d.num_pages, d.num_idx_heads, d.block_size, d.idx_dim)),
            _ptr(q, BF16, "q", (B, Hq, d.head_dim)), _ptr(k_cache, BF16, "k_cache", cache),
            _ptr(v_cache, BF16, "v_cache", cache),
            _ptr(block_table, I32, "block_table", (B, d.max_blocks_per_seq)),
            _ptr(seq_lens, I32, "seq_lens", (B,)),
            _ptr(out, BF16, "out", (B, Hq, d.head_dim)),
            _ptr(lse, F32, "lse", (B, Hq)) if lse is not None else None,
            _ptr(sel, I32, "sel", (B, H, d.topk)) if sel is not None else None,
            _ptr(workspace, torch.uint8, "workspace"))
    nbytes = workspace.numel() if workspace is not None else 0
    return PreparedCall(lib().msa_decode_step_append, (ctypes.byref(d), *args, nbytes),
                        "msa_decode_step_append",
                        (d, k_new, v_new, kidx_new, q_idx, kidx_cache, q, k_cache, v_cache,
                         block_table, seq_lens, out, lse, sel, workspace))


def msa_decode_step_append(dims, k_new, v_new, kidx_new, q_idx, kidx_cache, q, k_cache, v_cache,
                           block_table, seq_lens, out, lse, sel, workspace, stream=None):
    prepare_msa_decode_step_append(dims, k_new, v_new, kidx_new, q_idx, kidx_cache, q, k_cache,
                                   v_cache, block_table, seq_lens, out, lse, sel, workspace)(stream)


def msa_dense_decode_workspace_size(dims) -> int:
    return int(lib().msa_dense_decode_workspace_size(ctypes.byref(dims)))


def prepare_msa_dense_attn_decode(dims, q, k_cache, v_cache, block_table, seq_lens, out, lse,
                                  workspace):
    """msa_dense_attn_decode with its arguments checked and packed once: returns a
    PreparedCall that repeats the call, on the current (or a given) stream."""
    d = dims
    B, Hq, H = d.num_seqs, d.num_q_heads, d.num_kv_heads
    cache = (d.num_pages, H, d.block_size, d.head_dim)
    args = (_ptr(q, BF16, "q", (B, Hq, d.head_dim)), _ptr(k_cache, BF16, "k_cache", cache),
            _ptr(v_cache, BF16, "v_cache", cache),
            _ptr(block_table, I32, "block_table", (B, d.max_blocks_per_seq)),
            _ptr(seq_lens, I32, "seq_lens", (B,)),
            _ptr(out, BF16, "out", (B, Hq, d.head_dim)),
            _ptr(lse, F32, "lse", (B, Hq)) if lse is not None else None,
            _ptr(workspace, torch.uint8, "workspace"))
    nbytes = workspace.numel() if workspace is not None else 0
    return PreparedCall(lib().msa_dense_attn_decode, (ctypes.byref(d), *args, nbytes),
                        "msa_dense_attn_decode",
                        (d, q, k_cache, v_cache, block_table, seq_lens, out, lse, workspace))


def msa_dense_attn_decode(dims, q, k_cache, v_cache, block_table, seq_lens, out, lse, workspace,
                          stream=None):
    """Dense GQA decode over every cached token (the comparison baseline)."""
    prepare_msa_dense_attn_decode(dims, q, k_cache, v_cache, block_table, seq_lens, out, lse,
                                  workspace)(stream)


def prepare_msa_dense_attn_prefill(dims, total_q, q, k_cache, v_cache, block_table, seq_lens, cu_q,
                                   out, lse):
    """msa_dense_attn_prefill with its arguments checked and packed once: returns a
    PreparedCall that repeats the call, on the current (or a given) stream."""
    d = dims
    B, Hq, H = d.num_seqs, d.num_q_heads, d.num_kv_heads
    cache = (d.num_pages, H, d.block_size, d.head_dim)
    args = (_ptr(q, BF16, "q", (total_q, Hq, d.head_dim)), _ptr(k_cache, BF16, "k_cache", cache),
            _ptr(v_cache, BF16, "v_cache", cache),
            _ptr(block_table, I32, "block_table", (B, d.max_blocks_per_seq)),
            _ptr(seq_lens, I32, "seq_lens", (B,)), _ptr(cu_q, I32, "cu_q", (B + 1,)),
            _ptr(out, BF16, "out", (total_q, Hq, d.head_dim)),
            _ptr(lse, F32, "lse", (total_q, Hq)) if lse is not None else None)
    return PreparedCall(lib().msa_dense_attn_prefill, (ctypes.byref(d), total_q, *args),
                        "msa_dense_attn_prefill",
                        (d, q, k_cache, v_cache, block_table, seq_lens, cu_q, out, lse))


def msa_dense_attn_prefill(dims, total_q, q, k_cache, v_cache, block_table, seq_lens, cu_q, out,
                           lse, stream=None):
    """Dense causal attention over every cached token (the prefill baseline)."""
    prepare_msa_dense_attn_prefill(dims, total_q, q, k_cache, v_cache, block_table, seq_lens, cu_q,
                                   out, lse)(stream)


def prepare_msa_append_kv(dims, total_q, k_new, v_new, kidx_new, block_table, seq_lens, cu_q,
                          k_cache, v_cache, kidx_cache):
    """msa_append_kv with its arguments checked and packed once: returns a
    PreparedCall that repeats the call, on the current (or a given) stream."""
    d = dims
    B, H = d.num_seqs, d.num_kv_heads
    cache = (d.num_pages, H, d.block_size, d.head_dim)
    icache = (d.num_pages, d.num_idx_heads, d.block_size, d.idx_dim)
    args = (_ptr(k_new, BF16, "k_new", (total_q, H, d.head_dim)),
            _ptr(v_new, BF16, "v_new", (total_q, H, d.head_dim)),
            _ptr(kidx_new, BF16, "kidx_new", (total_q, d.num_idx_heads, d.idx_dim)),
            _ptr(block_table, I32, "block_table", (B, d.max_blocks_per_seq)),
            _ptr(seq_lens, I32, "seq_lens", (B,)), _ptr(cu_q, I32, "cu_q", (B + 1,)),
            _ptr(k_cache, BF16, "k_cache", cache), _ptr(v_cache, BF16, "v_cache", cache),
            _ptr(kidx_cache, BF16, "kidx_cache", icache))
    return PreparedCall(lib().msa_append_kv, (ctypes.byref(d), total_q, *args), "msa_append_kv",
                        (d, k_new, v_new, kidx_new, block_table, seq_lens, cu_q, k_cache,
                         v_cache, kidx_cache))


def msa_append_kv(dims, total_q, k_new, v_new, kidx_new, block_table, seq_lens, cu_q, k_cache,
                  v_cache, kidx_cache, stream=None):
    """The new tokens' K, V and index keys into their pages (include/msa.h)."""
    prepare_msa_append_kv(dims, total_q, k_new, v_new, kidx_new, block_table, seq_lens, cu_q,
                          k_cache, v_cache, kidx_cache)(stream)


MSA_FAULT_SEQ_LEN, MSA_FAULT_CU_Q, MSA_FAULT_BLOCK_TABLE = 1, 2, 4


def prepare_msa_validate_inputs(dims, total_q, block_table, seq_lens, cu_q, status):
    """msa_validate_inputs with its arguments checked and packed once: returns a
    PreparedCall that repeats the call, on the current (or a given) stream."""
    d = dims
    B = d.num_seqs
    args = (_ptr(block_table, I32, "block_table", (B, d.max_blocks_per_seq)),
            _ptr(seq_lens, I32, "seq_lens", (B,)),
            _ptr(cu_q, I32, "cu_q", (B + 1,)) if cu_q is not None else None,
            _ptr(status, I32, "status", (1,)))
    return PreparedCall(lib().msa_validate_inputs, (ctypes.byref(d), total_q, *args),
                        "msa_validate_inputs", (d, block_table, seq_lens, cu_q, status))


def msa_validate_inputs(dims, total_q, block_table, seq_lens, cu_q, status, stream=None):
    """Device-side check of the content preconditions; `status` (one int32 on
    the device) receives 0 or the OR of the MSA_FAULT_* bits found."""
    prepare_msa_validate_inputs(dims, total_q, block_table, seq_lens, cu_q, status)(stream)
