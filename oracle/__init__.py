"""fp64 CPU oracle for MiniMax Sparse Attention (MSA) -- test infrastructure.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library
(``block_sparse_attention_03_amd``) never imports it and shares no code with
it; the only thing both sides share is the seeded input generator module,
which holds none of the method's arithmetic.

The arithmetic lives in ``msa_oracle.c`` (plain C, fp64, OpenMP over rows);
this module only builds it with gcc and marshals numpy arrays.  Each wrapper
cites the passage it follows in the C file's comments.  The one exception is
the cache append, a plain copy into the slots of the positions that the C
code computes, written here with numpy indexing.  bf16 tensors are
passed as ``uint16`` arrays of raw bits.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "msa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmsa_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
               "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or (
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int
        L = ctypes.c_long
        D = ctypes.c_double
        lib.msa_oracle_threads.restype = I
        lib.msa_oracle_positions.argtypes = [I, P, P, P, P]
        lib.msa_oracle_positions.restype = I
        lib.msa_oracle_index_score.argtypes = [I, I, I, I, I, I, P, P, P, P, P, L, P, P]
        lib.msa_oracle_topk.argtypes = [L, I, I, P, P, P]
        lib.msa_oracle_attention.argtypes = [I, I, I, I, I, I, I, D, P, P, P, P, P, P, P,
                                             L, P, P, P]
        lib.msa_oracle_page_table.argtypes = [I, I, I, I, I, P, P, P, P, P]
        lib.msa_oracle_paged_attention.argtypes = [I, I, I, I, I, I, D, P, P, P, P, P, P, P]
        lib.msa_oracle_lse_merge.argtypes = [L, I, I, P, P, P, P]
        _lib = lib
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def threads() -> int:
    """OpenMP threads the oracle uses (OMP_NUM_THREADS, else all cores)."""
    return int(_load().msa_oracle_threads())


def positions(seq_lens, cu_q):
    """(seq_of[T], pos_of[T]): p = L_s - n_s + i for the i-th new token of s."""
    seq_lens = _c(seq_lens, np.int32)
    cu_q = _c(cu_q, np.int32)
    B = seq_lens.shape[0]
    T = int(cu_q[-1])
    seq_of = np.zeros(max(T, 1), np.int32)
    pos_of = np.zeros(max(T, 1), np.int32)
    rc = _load().msa_oracle_positions(B, _p(seq_lens), _p(cu_q), _p(seq_of), _p(pos_of))
    if rc != 0:
        raise ValueError("a sequence has more query tokens than cache tokens")
    return seq_of[:T], pos_of[:T]


def append_kv(k_cache, v_cache, kidx_cache, k_new, v_new, kidx_new, block_table, seq_lens,
              cu_q, block_size):
    """Cache append by its definition ([aivizor] paragraph on MSA with paged
    attention: paged caches, one page per block): the i-th new token of
    sequence s, at position p = seq_lens[s] - n_s + i, goes to page
    block_table[s][p // block_size], slot p % block_size, for every KV group
    (K, V) and index head (k_idx).  Works on raw bf16 bits; returns updated
    copies of the three caches."""
    seq_of, pos_of = positions(seq_lens, cu_q)
    K, V, I = k_cache.copy(), v_cache.copy(), kidx_cache.copy()
    for t in range(len(seq_of)):
        s, p = int(seq_of[t]), int(pos_of[t])
        page = int(block_table[s][p // block_size])
        K[page, :, p % block_size, :] = k_new[t]
        V[page, :, p % block_size, :] = v_new[t]
        I[page, :, p % block_size, :] = kidx_new[t]
    return K, V, I


def index_score(q_idx, kidx_cache, block_table, seq_of, pos_of, block_size, rows=None):
    """fp64 block scores [n_rows, maxblk] (rows: flat t*H_kv+g, default all)."""
    q_idx = _c(q_idx, np.uint16)
    kidx_cache = _c(kidx_cache, np.uint16)
    block_table = _c(block_table, np.int32)
    T, H_kv, d = q_idx.shape
    H_idx = kidx_cache.shape[1]
    maxblk = block_table.shape[1]
    rows_a = None if rows is None else _c(rows, np.int64)
    n = T * H_kv if rows is None else rows_a.shape[0]
    out = np.empty((n, maxblk), np.float64)
    _load().msa_oracle_index_score(T, H_kv, H_idx, d, block_size, maxblk, _p(q_idx),
                                   _p(kidx_cache), _p(block_table), _p(_c(seq_of, np.int32)),
                                   _p(_c(pos_of, np.int32)), n, _p(rows_a), _p(out))
    return out


def topk(scores, b_loc, k):
    """Selection [n_rows, k] from scores [n_rows, maxblk] and per-row b_loc."""
    scores = _c(scores, np.float64)
    b_loc = _c(b_loc, np.int32)
    n, maxblk = scores.shape
    if n and int(b_loc.max()) >= maxblk:
        raise ValueError("b_loc beyond the score width")
    sel = np.empty((n, k), np.int32)
    _load().msa_oracle_topk(n, maxblk, k, _p(scores), _p(b_loc), _p(sel))
    return sel


def attention(q, k_cache, v_cache, block_table, seq_of, pos_of, sel, scale=None, rows=None):
    """(out [n_rows, D] fp64, lse [n_rows]) over the selected blocks' tokens.

    rows are flat t*H_q+h (default all); sel is [T, H_kv, k].
    """
    q = _c(q, np.uint16)
    k_cache = _c(k_cache, np.uint16)
    v_cache = _c(v_cache, np.uint16)
    block_table = _c(block_table, np.int32)
    sel = _c(sel, np.int32)
    T, H_q, D = q.shape
    H_kv, Bk = k_cache.shape[1], k_cache.shape[2]
    k = sel.shape[2]
    maxblk = block_table.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    rows_a = None if rows is None else _c(rows, np.int64)
    n = T * H_q if rows is None else rows_a.shape[0]
    out = np.empty((n, D), np.float64)
    lse = np.empty(n, np.float64)
    _load().msa_oracle_attention(T, H_q, H_kv, D, Bk, k, maxblk, float(scale), _p(q),
                                 _p(k_cache), _p(v_cache), _p(block_table),
                                 _p(_c(seq_of, np.int32)), _p(_c(pos_of, np.int32)), _p(sel),
                                 n, _p(rows_a), _p(out), _p(lse))
    return out, lse


def page_table(sel, block_table, seq_lens, block_size):
    """Decode page table [B*H_kv, k] and row lengths [B*H_kv] from sel [B, H_kv, k]."""
    sel = _c(sel, np.int32)
    block_table = _c(block_table, np.int32)
    seq_lens = _c(seq_lens, np.int32)
    B, H_kv, k = sel.shape
    pt = np.empty((B * H_kv, k), np.int32)
    rl = np.empty(B * H_kv, np.int32)
    _load().msa_oracle_page_table(B, H_kv, k, block_size, block_table.shape[1], _p(sel),
                                  _p(block_table), _p(seq_lens), _p(pt), _p(rl))
    return pt, rl


def paged_attention(q, k_cache, v_cache, page_table_, row_lens, scale=None):
    """Fixed-page attention over the flattened batch; q is [B, H_q, D]."""
    q = _c(q, np.uint16)
    k_cache = _c(k_cache, np.uint16)
    v_cache = _c(v_cache, np.uint16)
    page_table_ = _c(page_table_, np.int32)
    row_lens = _c(row_lens, np.int32)
    B, H_q, D = q.shape
    H_kv, Bk = k_cache.shape[1], k_cache.shape[2]
    G = H_q // H_kv
    R = B * H_kv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.empty((R * G, D), np.float64)
    lse = np.empty(R * G, np.float64)
    _load().msa_oracle_paged_attention(R, G, H_kv, D, Bk, page_table_.shape[1], float(scale),
                                       _p(q), _p(k_cache), _p(v_cache), _p(page_table_),
                                       _p(row_lens), _p(out), _p(lse))
    return out.reshape(B, H_q, D), lse.reshape(B, H_q)


def lse_merge(o_parts, lse_parts):
    """Merge partials o_parts [n, parts, D], lse_parts [n, parts] -> (o, lse)."""
    o_parts = _c(o_parts, np.float64)
    lse_parts = _c(lse_parts, np.float64)
    n, parts, D = o_parts.shape
    o = np.empty((n, D), np.float64)
    lse = np.empty(n, np.float64)
    _load().msa_oracle_lse_merge(n, parts, D, _p(o_parts), _p(lse_parts), _p(o), _p(lse))
    return o, lse


def b_loc_rows(pos_of, H_kv, block_size, rows=None):
    """Own block of each flat (t*H_kv+g) row -- the query position over Bk."""
    pos = np.asarray(pos_of, np.int64)
    r = np.arange(pos.shape[0] * H_kv) if rows is None else np.asarray(rows, np.int64)
    return (pos[r // H_kv] // block_size).astype(np.int32)
