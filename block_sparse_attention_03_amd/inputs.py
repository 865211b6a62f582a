"""Seeded synthetic inputs for the MSA hot path.

This module is shared by the HIP path's tests/bench and by the oracle's
tests.  It holds none of the method's arithmetic: it only draws values,
lengths, page permutations and per-block key scales, and lays them out in the
tensor formats the library takes.

Workload shapes follow the pages' own workloads:
  * decode at 4k context, batch 1, GQA 4 (a small case);
  * paged decode at concurrency 8 over a 60,000-token cached prefix (the
    agentic-traffic measurement in the aivizor serving-report news item),
    physical pages randomly permuted, keys given a per-block scale so that
    block scores spread;
  * chunked prefill of 8192 new tokens onto a 57,344-token prefix (the
    chunked-prefill size of the SGLang launch command in the mechatronicstore
    "MoE de 428B con 1M de contexto" page);
  * decode at a 1M-token context (the context window in both the aivizor and
    mechatronicstore pages);
  * ragged decode over 16 sequences with log-uniform context lengths.
All share head_dim 128, idx_dim 64, Bk = 128, k = 16 (youmind page, bullet
"Costo predecible a cualquier longitud").

Values are bf16 drawn as fp32 N(0,1) from a torch.Generator seeded per
config on the target device, then rounded to nearest-even bf16.  Host-side
metadata (lengths, permutations, key scales) come from numpy's default_rng
with the same seed, so they do not depend on the device.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np
import torch


@dataclasses.dataclass
class MsaConfig:
    name: str
    seq_lens: List[int]          # cache tokens per sequence, new tokens included
    n_new: List[int]             # query tokens per sequence (1 in decode)
    num_q_heads: int
    num_kv_heads: int
    num_idx_heads: int = 1       # 1 = shared index key per token, or num_kv_heads
    head_dim: int = 128
    idx_dim: int = 64
    block_size: int = 128
    topk: int = 16
    permute_pages: bool = False
    key_block_scale: bool = False
    extra_pages: int = 0         # spare pool pages nobody references
    seed: int = 0

    @property
    def num_seqs(self) -> int:
        return len(self.seq_lens)

    @property
    def total_q(self) -> int:
        return int(sum(self.n_new))

    @property
    def blocks_per_seq(self) -> List[int]:
        return [(L + self.block_size - 1) // self.block_size for L in self.seq_lens]

    @property
    def max_blocks(self) -> int:
        return max(self.blocks_per_seq) if self.seq_lens else 1

    @property
    def num_pages(self) -> int:
        return sum(self.blocks_per_seq) + self.extra_pages

    @property
    def is_decode(self) -> bool:
        return all(n == 1 for n in self.n_new)

    def with_idx_heads(self, h: int) -> "MsaConfig":
        return dataclasses.replace(self, num_idx_heads=h, name=f"{self.name}_hidx{h}")


def _ragged_lengths(n: int, lo: int, hi: int, seed: int) -> List[int]:
    """Log-uniform integer lengths in [lo, hi]: u ~ U[ln lo, ln hi), L = round(e^u)."""
    rng = np.random.default_rng(seed + 1000)
    u = rng.uniform(math.log(lo), math.log(hi), size=n)
    return [int(min(max(round(math.exp(x)), lo), hi)) for x in u]


def config(i: int) -> MsaConfig:
    """The five workloads, numbered 1..5 as listed in the module docstring."""
    if i == 1:
        return MsaConfig("decode_b1_ctx4k", [4096], [1], 8, 2, seed=1)
    if i == 2:
        return MsaConfig("paged_decode_b8_ctx60k", [60000] * 8, [1] * 8, 48, 8,
                         permute_pages=True, key_block_scale=True, seed=2)
    if i == 3:
        return MsaConfig("chunked_prefill_8k_on_57k", [65536], [8192], 48, 8, seed=3)
    if i == 4:
        return MsaConfig("decode_b4_ctx1m", [1048576] * 4, [1] * 4, 64, 8, seed=4)
    if i == 5:
        return MsaConfig("ragged_decode_16seq", _ragged_lengths(16, 4096, 524288, 5),
                         [1] * 16, 48, 8, permute_pages=True, seed=5)
    raise ValueError(f"no workload {i}")


@dataclasses.dataclass
class MsaInputs:
    cfg: MsaConfig
    q_idx: torch.Tensor        # [T, H_kv, d] bf16
    q: torch.Tensor            # [T, H_q, D] bf16
    kidx_cache: torch.Tensor   # [P, H_idx, Bk, d] bf16
    k_cache: torch.Tensor      # [P, H_kv, Bk, D] bf16
    v_cache: torch.Tensor      # [P, H_kv, Bk, D] bf16
    block_table: torch.Tensor  # [B, maxblk] int32 (unused entries point at page 0)
    seq_lens: torch.Tensor     # [B] int32
    cu_q: torch.Tensor         # [B+1] int32


def _randn_bf16(shape, gen, device, chunk_rows: int = 4096) -> torch.Tensor:
    """N(0,1) fp32 draws rounded to bf16, generated in row chunks (bounded memory)."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    n0 = shape[0]
    for a in range(0, n0, chunk_rows):
        b = min(n0, a + chunk_rows)
        out[a:b] = torch.randn((b - a,) + tuple(shape[1:]), generator=gen,
                               dtype=torch.float32, device=device).to(torch.bfloat16)
    return out


def make_inputs(cfg: MsaConfig, device="cpu", poison_padding: bool = False) -> MsaInputs:
    """Draw every tensor of ``cfg`` on ``device``.

    poison_padding writes NaN into the cache slots past each sequence's last
    token (k_idx, K and V), which the method must never read into a result.
    """
    device = torch.device(device)
    rng = np.random.default_rng(cfg.seed)
    B, Bk = cfg.num_seqs, cfg.block_size
    nblk = cfg.blocks_per_seq
    maxblk = cfg.max_blocks
    P = cfg.num_pages

    # logical block (s, b) -> physical page
    order = rng.permutation(P) if cfg.permute_pages else np.arange(P)
    bt = np.zeros((B, maxblk), np.int32)
    off = 0
    for s in range(B):
        bt[s, :nblk[s]] = order[off:off + nblk[s]]
        off += nblk[s]

    gen = torch.Generator(device=device)
    gen.manual_seed(cfg.seed)
    T = cfg.total_q
    q_idx = _randn_bf16((T, cfg.num_kv_heads, cfg.idx_dim), gen, device)
    q = _randn_bf16((T, cfg.num_q_heads, cfg.head_dim), gen, device)
    kidx = _randn_bf16((P, cfg.num_idx_heads, Bk, cfg.idx_dim), gen, device, 1024)
    kc = _randn_bf16((P, cfg.num_kv_heads, Bk, cfg.head_dim), gen, device, 256)
    vc = _randn_bf16((P, cfg.num_kv_heads, Bk, cfg.head_dim), gen, device, 256)

    if cfg.key_block_scale:
        # one scale per (sequence, logical block), applied in fp32 to both kinds
        # of key (K and k_idx) of that block, then rounded back to bf16
        scale = np.ones(P, np.float32)
        for s in range(B):
            scale[bt[s, :nblk[s]]] = rng.uniform(0.5, 2.0, size=nblk[s]).astype(np.float32)
        sc = torch.from_numpy(scale).to(device)
        step = 1024
        for a in range(0, P, step):
            b = min(P, a + step)
            kidx[a:b] = (kidx[a:b].float() * sc[a:b, None, None, None]).to(torch.bfloat16)
            kc[a:b] = (kc[a:b].float() * sc[a:b, None, None, None]).to(torch.bfloat16)

    if poison_padding:
        nan = float("nan")
        for s in range(B):
            tail = cfg.seq_lens[s] % Bk
            if tail:
                page = int(bt[s, nblk[s] - 1])
                kidx[page, :, tail:, :] = nan
                kc[page, :, tail:, :] = nan
                vc[page, :, tail:, :] = nan

    cu = np.zeros(B + 1, np.int32)
    cu[1:] = np.cumsum(cfg.n_new)
    return MsaInputs(cfg, q_idx, q, kidx, kc, vc,
                     torch.from_numpy(bt).to(device),
                     torch.tensor(cfg.seq_lens, dtype=torch.int32, device=device),
                     torch.from_numpy(cu).to(device))


def bits(t: torch.Tensor) -> np.ndarray:
    """Host numpy view of a tensor's raw bits (bf16 -> uint16)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
