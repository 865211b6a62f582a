"""Algorithmic work of one MSA layer-step: bytes and flops the method must move.

Counts cover only what the method has to touch -- index keys of every valid
context token, K and V of the attended tokens, the small per-query vectors --
and never the dense work that MSA avoids, nor padding or re-reads.  They are
the numerators of the roofline fractions bench.py reports.
"""
from __future__ import annotations

import math


def _attended(cfg):
    """Per (query token) list of (position p, attended tokens per group).

    With top-k over blocks 0..b_loc, a query attends min(k, b_loc+1) blocks:
    all but its own are full, its own holds p - Bk*b_loc + 1 visible tokens.
    """
    Bk, k = cfg.block_size, cfg.topk
    out = []
    for L, n in zip(cfg.seq_lens, cfg.n_new):
        for i in range(n):
            p = L - n + i
            b_loc = p // Bk
            n_sel = min(k, b_loc + 1)
            out.append((p, (n_sel - 1) * Bk + (p - Bk * b_loc + 1)))
    return out


def score_bytes(cfg) -> int:
    """Index scoring: every visible token's index key once per index head, the
    index queries, and the eligible block scores written (fp32)."""
    kidx = sum(cfg.seq_lens) * cfg.num_idx_heads * cfg.idx_dim * 2
    qidx = cfg.total_q * cfg.num_kv_heads * cfg.idx_dim * 2
    sc = sum((p // cfg.block_size + 1) for p, _ in _attended(cfg)) * cfg.num_kv_heads * 4
    return kidx + qidx + sc


def score_flops(cfg) -> int:
    """2*d*H_kv flops per (query, visible context token)."""
    return sum(2 * cfg.idx_dim * cfg.num_kv_heads * (p + 1) for p, _ in _attended(cfg))


def decode_attn_bytes(cfg) -> int:
    """K and V of the attended tokens of every (sequence, group) row, q read,
    out written (bf16) and lse written (fp32)."""
    D = cfg.head_dim
    kv = sum(n_att for _, n_att in _attended(cfg)) * cfg.num_kv_heads * 2 * D * 2
    qo = cfg.total_q * cfg.num_q_heads * (2 * D * 2 + 4)
    return kv + qo


def attn_flops(cfg) -> int:
    """4*D flops per (query, head, attended token): q.k and p*v."""
    return sum(4 * cfg.head_dim * cfg.num_q_heads * n_att for _, n_att in _attended(cfg))


def dense_prefill_flops(cfg) -> int:
    """Dense causal baseline: the query at position p attends p + 1 tokens."""
    n = 0
    for L, q in zip(cfg.seq_lens, cfg.n_new):
        # positions L-q .. L-1 attend L-q+1 .. L tokens
        n += q * (L - q) + q * (q + 1) // 2
    return 4 * cfg.head_dim * cfg.num_q_heads * n


def prefill_attn_bytes(cfg) -> int:
    """KV-block-major prefill: each selected (sequence, group, block) K and V
    once, q read once per (query, head, slot), out + lse written, and the
    partial outputs (bf16) and LSEs (fp32) written and read back once."""
    D, Bk = cfg.head_dim, cfg.block_size
    G = cfg.num_q_heads // cfg.num_kv_heads
    blocks = 0
    for L, n in zip(cfg.seq_lens, cfg.n_new):
        if n:
            blocks += (L - 1) // Bk + 1  # upper bound: every block is selected by someone
    kv = blocks * cfg.num_kv_heads * 2 * Bk * D * 2
    slots = sum(min(cfg.topk, p // Bk + 1) for p, _ in _attended(cfg)) * cfg.num_kv_heads * G
    q = slots * D * 2
    partial = slots * (D * 2 + 4) * 2
    out = cfg.total_q * cfg.num_q_heads * (D * 2 + 4)
    return kv + q + partial + out


def multi_query_attn_bytes(cfg, sel) -> int:
    """Few queries per sequence, block-major over each (sequence, group)'s
    union of selected blocks (sel: [total_q, H_kv, k] block indices, -1 for
    none, the call's own selection): K and V of every block in a union once
    (its tokens up to the sequence end), q read once per (query, head, slot),
    the partial outputs (bf16) and LSEs (fp32) written and read back once,
    out + lse written."""
    D, Bk = cfg.head_dim, cfg.block_size
    G = cfg.num_q_heads // cfg.num_kv_heads
    kv_tokens = 0
    slots = 0
    t = 0
    for L, n in zip(cfg.seq_lens, cfg.n_new):
        for g in range(cfg.num_kv_heads):
            union = set()
            for i in range(n):
                row = [int(b) for b in sel[t + i][g] if b >= 0]
                union.update(row)
                slots += len(row)
            kv_tokens += sum(min(Bk, L - b * Bk) for b in union)
        t += n
    kv = kv_tokens * 2 * D * 2
    q = slots * G * D * 2
    partial = slots * G * (D * 2 + 4) * 2
    out = cfg.total_q * cfg.num_q_heads * (D * 2 + 4)
    return kv + q + partial + out


def dense_over_msa_flops(L: int, num_q_heads: int, num_idx_q_heads: int, head_dim: int = 128,
                         idx_dim: int = 64, budget: int = 2048) -> float:
    """Attention flops per token of dense GQA over those of MSA at context L.

    Dense: 4*D*H_q*L.  MSA: 4*D*H_q*budget (attention over the selected
    tokens) + 2*d*H_idxq*L (index scoring over the whole context).
    """
    dense = 4 * head_dim * num_q_heads * L
    msa = 4 * head_dim * num_q_heads * min(budget, L) + 2 * idx_dim * num_idx_q_heads * L
    return dense / msa


HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix, published
