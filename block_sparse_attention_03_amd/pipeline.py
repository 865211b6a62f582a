"""One MSA layer-step through the C ABI, with its device buffers.

Decode:  msa_index_score -> msa_topk_blocks -> msa_build_page_table ->
         msa_sparse_attn_decode, or the fused msa_decode_step (same results).
Prefill: msa_index_score -> msa_topk_blocks -> msa_sparse_attn_prefill, or the
         one msa_multi_query_step call (same results).
This module only allocates the outputs and the workspace (torch device memory)
and calls the library; every step of the computation runs in its kernels.
"""
from __future__ import annotations

import torch

from . import _lib as L


class MsaStep:
    def __init__(self, x, lse: bool = True, fused: bool = False, prefill: bool = False,
                 multi: bool = False):
        """fused: the decode step as one msa_decode_step call; prefill: take the
        prefill entry point even when every sequence has a single query; multi:
        the prefill path as one msa_multi_query_step call."""
        cfg = x.cfg
        self.x = x
        self.cfg = cfg
        self.dims = L.dims_for(cfg)
        dev = x.q.device
        T, H, W = cfg.total_q, cfg.num_kv_heads, cfg.max_blocks
        self.decode = cfg.is_decode and not prefill
        self.scores = torch.empty((T, H, W), dtype=torch.float32, device=dev)
        self.sel = torch.empty((T, H, cfg.topk), dtype=torch.int32, device=dev)
        self.out = torch.empty((T, cfg.num_q_heads, cfg.head_dim), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((T, cfg.num_q_heads), dtype=torch.float32, device=dev) if lse else None
        self.fused = fused and self.decode
        self.multi = multi and not self.decode
        if self.fused:
            nbytes = L.msa_decode_step_workspace_size(self.dims)
        elif self.multi:
            nbytes = L.msa_multi_query_step_workspace_size(self.dims, T)
        elif self.decode:
            R = cfg.num_seqs * H
            self.page_table = torch.empty((R, cfg.topk), dtype=torch.int32, device=dev)
            self.row_lens = torch.empty((R,), dtype=torch.int32, device=dev)
            nbytes = L.msa_decode_workspace_size(self.dims)
        else:
            nbytes = L.msa_prefill_workspace_size(self.dims, T)
        if nbytes == 0:
            raise L.MsaError(L.MSA_ERROR_NOT_SUPPORTED, "workspace size")
        self.workspace = torch.empty((nbytes,), dtype=torch.uint8, device=dev)

        # every call's arguments checked and packed once (the buffers above
        # and the inputs' tensors are reused by every run)
        self._score = L.prepare_msa_index_score(self.dims, T, x.q_idx, x.kidx_cache,
                                                x.block_table, x.seq_lens, x.cu_q, self.scores)
        self._topk = L.prepare_msa_topk_blocks(self.dims, T, self.scores, x.seq_lens, x.cu_q,
                                               self.sel)
        if self.fused:
            self._fused = L.prepare_msa_decode_step(self.dims, x.q_idx, x.kidx_cache, x.q,
                                                    x.k_cache, x.v_cache, x.block_table,
                                                    x.seq_lens, self.out, self.lse, self.sel,
                                                    self.workspace)
        elif self.multi:
            self._fused = L.prepare_msa_multi_query_step(self.dims, T, x.q_idx, x.kidx_cache, x.q,
                                                         x.k_cache, x.v_cache, x.block_table,
                                                         x.seq_lens, x.cu_q, self.out, self.lse,
                                                         self.sel, self.workspace)
        elif self.decode:
            self._page_table = L.prepare_msa_build_page_table(self.dims, self.sel, x.block_table,
                                                              x.seq_lens, self.page_table,
                                                              self.row_lens)
            self._attend = L.prepare_msa_sparse_attn_decode(self.dims, x.q, x.k_cache, x.v_cache,
                                                            self.page_table, self.row_lens,
                                                            self.out, self.lse, self.workspace)
        else:
            self._attend = L.prepare_msa_sparse_attn_prefill(self.dims, T, x.q, x.k_cache,
                                                             x.v_cache, x.block_table, x.seq_lens,
                                                             x.cu_q, self.sel, self.out, self.lse,
                                                             self.workspace)

    def score(self, stream=None):
        self._score(stream)

    def topk(self, stream=None):
        self._topk(stream)

    def page_table_step(self, stream=None):
        self._page_table(stream)

    def attend(self, stream=None):
        self._attend(stream)

    def fused_step(self, stream=None):
        self._fused(stream)

    def run(self, stream=None):
        if self.fused or self.multi:
            self.fused_step(stream)
            return self.out
        self.score(stream)
        self.topk(stream)
        if self.decode:
            self.page_table_step(stream)
        self.attend(stream)
        return self.out
