"""Row widths and edge cases that pick distinct kernel instantiations (needs an
MI355X; every call goes through the C ABI).

The selection kernels are compiled per row width (max_blocks_per_seq):

  width        msa_topk_blocks            msa_decode_step (fused selection)
  <= 256       topk_kernel<8, 1>          decode_fused_kernel<4, 1, true>
  257..512     topk_kernel<8, 1>          decode_fused_kernel<8, 1, true>
  513..1024    topk_kernel<16, 1>         decode_fused_kernel<16, 1, true>
  1025..2048   topk_kernel<8, 4>          decode_fused_kernel<8, 4, true>
  2049..4096   topk_kernel<8, 8>          decode_fused_kernel<16, 4, true>
  4097..8192   topk_kernel<8, 16>         decode_fused_kernel<32, 4, false>
  8193..16384  topk_kernel<16, 16>        standalone selection + page kernels

The width is the batch's widest row, so a short row in a wide batch runs the
wide form with most of its candidate slots empty.  The cases here put a long
and a short row in each band; each goes through the four calls (checked
against the oracle, padding poisoned with NaN) and through msa_decode_step
(bit-equal to the four calls).

msa_decode_step also picks, by the number of flattened rows R (sequences x
KV groups), how many page slots one workgroup attends: one while all 16 R
page workgroups fit on the chip at once (R <= 64), else 2, 4 or 8
(decode_multi_kernel<NPT, W, PAGES, slots>: R < 128, R < 256, R >= 256).
MULTI covers each of those with short and long rows.

msa_sparse_attn_prefill picks its form by the number of queries T, the
batch size B and the row width: with T x k <= 4096 and T <= 32 B (draft
tokens, a few dozen per sequence at most) mq_block_kernel finds each
(sequence, group)'s union of selected blocks itself and attends each block
once for all the queries that chose it; otherwise an inverse map (one
workgroup while the buckets and selections are few, else four kernels) feeds
the block-major kernel (buckets of more than 32 rows) and the small-bucket
kernel.  MQ covers the first form's limits and both switches.
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_03_amd import inputs as gen
from block_sparse_attention_03_amd.pipeline import MsaStep

import parity

pytestmark = pytest.mark.gpu

BANDS = [
    # 513..1024 blocks: 16 candidates per lane, one selecting wavefront
    gen.MsaConfig("band_600_blocks", [76_800, 3_000], [1, 1], 8, 2, permute_pages=True, seed=81),
    gen.MsaConfig("band_782_blocks", [100_000, 70_000, 3_000], [1, 1, 1], 12, 3,
                  permute_pages=True, seed=82),
    gen.MsaConfig("band_1024_blocks", [131_072, 700], [1, 1], 8, 2, permute_pages=True, seed=83),
    # 4097..8192 blocks: the 16-wavefront selection and the four-wavefront
    # fused selection without block-table loads, rows partly filled
    gen.MsaConfig("band_5469_blocks", [700_000, 530_000, 9_000], [1, 1, 1], 4, 2,
                  permute_pages=True, seed=84),
    gen.MsaConfig("band_6000_blocks", [6000 * 128 - 77, 5_000], [1, 1], 6, 1,
                  permute_pages=True, seed=85),
    gen.MsaConfig("band_8192_blocks_1m_and_5k", [1_048_576, 5_000], [1, 1], 2, 1,
                  permute_pages=True, seed=86),
]


@pytest.mark.parametrize("cfg", BANDS, ids=lambda c: c.name)
def test_selection_width_bands(cfg):
    print(f"[band] {cfg.name} maxblk={cfg.max_blocks} lens={cfg.seq_lens}", flush=True)
    x, step = parity.full_check(cfg, poison=True)
    fused = MsaStep(x, fused=True)
    fused.sel.fill_(-7)
    fused.run()
    torch.cuda.synchronize()
    assert torch.equal(fused.sel, step.sel)
    assert torch.equal(fused.out, step.out)
    assert torch.equal(fused.lse, step.lse)


@pytest.mark.parametrize("n_new", [[130, 40], [3, 2]], ids=["inverse_map", "multi_query_form"])
def test_prefill_row_with_no_selection(n_new):
    """A (query, group) row of sel that is all -1 attends no token: its heads
    get out = 0 and lse = -inf, as the oracle defines the empty token set;
    the other rows are unchanged and match the oracle.  Both forms of the
    prefill entry point: the inverse map (170 queries) and the few-query
    kernel (5 queries)."""
    import oracle
    cfg = gen.MsaConfig(f"prefill_empty_rows_{sum(n_new)}", [2600, 900], n_new, 12, 3,
                        permute_pages=True, seed=87)
    print(f"[empty-row] {cfg.name}", flush=True)
    x = gen.make_inputs(cfg, device="cuda", poison_padding=True)
    step = MsaStep(x)
    step.score()
    step.topk()
    torch.cuda.synchronize()
    T, H, G = cfg.total_q, cfg.num_kv_heads, cfg.num_q_heads // cfg.num_kv_heads
    empty = sorted({(0, 0), (min(5, T - 1), 2), (min(129, T - 1), 1), (T - 1, 0), (T - 1, 2)})
    for t, g in empty:
        step.sel[t, g, :] = -1
    step.attend()
    torch.cuda.synchronize()
    seq_of, pos_of = oracle.positions(cfg.seq_lens, gen.bits(x.cu_q))
    sel = step.sel.cpu().numpy()
    kp, vp, bt2 = parity.compact_pages(x, sel, seq_of)
    ref_o, ref_l = oracle.attention(gen.bits(x.q), kp, vp, bt2, seq_of, pos_of, sel)
    got_o = step.out.reshape(T * cfg.num_q_heads, -1).float().cpu().numpy()
    got_l = step.lse.reshape(-1).cpu().numpy()
    is_empty = np.zeros(T * cfg.num_q_heads, bool)
    for t, g in empty:
        is_empty[t * cfg.num_q_heads + g * G: t * cfg.num_q_heads + (g + 1) * G] = True
    assert np.all(np.isneginf(ref_l[is_empty])) and np.all(ref_o[is_empty] == 0)
    assert np.all(got_o[is_empty] == 0), "empty rows: out must be 0"
    assert np.all(np.isneginf(got_l[is_empty])), "empty rows: lse must be -inf"
    ok = ~is_empty
    err = np.abs(got_o[ok] - ref_o[ok])
    assert (err <= parity.OUT_ATOL + parity.OUT_RTOL * np.abs(ref_o[ok])).all()
    assert np.abs(got_l[ok] - ref_l[ok]).max() <= parity.LSE_ATOL


def _lens(n, lo, hi, seed):
    rng = np.random.default_rng(seed)
    return [int(x) for x in rng.integers(lo, hi, size=n)]


MULTI = [
    # 96 rows: two slots per workgroup, one selecting wavefront
    gen.MsaConfig("multi_96_rows", _lens(12, 1_000, 40_000, 1), [1] * 12, 48, 8,
                  permute_pages=True, seed=94),
    # 72 rows with one 600,000-token row: two slots, four selecting
    # wavefronts without block-table loads (width 4688)
    gen.MsaConfig("multi_72_rows_600k", [600_000] + _lens(8, 500, 9_000, 2), [1] * 9, 16, 8,
                  permute_pages=True, seed=95),
    # 144 rows with a 300,000-token row: four slots, four selecting
    # wavefronts (width 2344)
    gen.MsaConfig("multi_144_rows_300k", [300_000] + _lens(17, 200, 12_000, 3), [1] * 18, 24, 8,
                  permute_pages=True, seed=96),
    # 256 rows: eight slots per workgroup
    gen.MsaConfig("multi_256_rows", _lens(32, 3_000, 20_000, 4), [1] * 32, 32, 8,
                  permute_pages=True, seed=97),
]


@pytest.mark.parametrize("cfg", MULTI, ids=lambda c: c.name)
def test_multi_page_workgroups(cfg):
    """Several page slots per workgroup in msa_decode_step: the four calls
    against the oracle, and the step bit-equal to them."""
    R = cfg.num_seqs * cfg.num_kv_heads
    print(f"[multi] {cfg.name} rows={R} maxblk={cfg.max_blocks}", flush=True)
    assert R * cfg.topk > 1024
    x, step = parity.full_check(cfg, poison=True, attn_rows=1024)
    fused = MsaStep(x, fused=True)
    fused.sel.fill_(-7)
    fused.run()
    torch.cuda.synchronize()
    assert torch.equal(fused.sel, step.sel)
    assert torch.equal(fused.out, step.out)
    assert torch.equal(fused.lse, step.lse)


MQ = [
    # 60 of the 64 queries in one sequence (its union spans many workgroups
    # of about eight blocks), a sequence with none
    gen.MsaConfig("mq_skewed_64", [30_000, 9_000, 5_000, 700], [60, 0, 3, 1], 48, 8,
                  permute_pages=True, seed=101),
    # 256 queries, all in one of 8 sequences (32 per sequence on average):
    # every entry slot of the kernel used by that sequence's groups
    gen.MsaConfig("mq_256_in_one_of_8", [20_000] + [3_000] * 7, [256] + [0] * 7, 16, 2,
                  permute_pages=True, seed=102),
    # 257 queries: past the kernel's entries, the one-workgroup inverse map
    gen.MsaConfig("mq_257_in_one_of_8", [20_000] + [3_000] * 7, [257] + [0] * 7, 16, 2,
                  permute_pages=True, seed=103),
    # 33 queries per sequence on average: the inverse map and bucket kernels
    gen.MsaConfig("mq_33_per_sequence", [16_000, 9_000], [33, 33], 16, 2, permute_pages=True,
                  seed=108),
    # 32 per sequence: still the multi-query kernel
    gen.MsaConfig("mq_32_per_sequence", [16_000, 9_000], [32, 32], 16, 2, permute_pages=True,
                  seed=109),
    # G = 1, drafts of several lengths
    gen.MsaConfig("mq_g1", [5_000, 12_000, 800], [4, 7, 2], 4, 4, permute_pages=True, seed=104),
    # a 2,097,152-token row (16,384 blocks: two bitmap words per thread)
    gen.MsaConfig("mq_2m_tokens", [16384 * 128, 3_000], [3, 2], 8, 1, permute_pages=True,
                  seed=105),
]


@pytest.mark.parametrize("cfg", MQ, ids=lambda c: c.name)
def test_multi_query_kernel(cfg):
    """Few queries per sequence through msa_sparse_attn_prefill: scores,
    selection and every attention row against the oracle, padding poisoned."""
    print(f"[mq] {cfg.name} T={cfg.total_q} maxblk={cfg.max_blocks}", flush=True)
    parity.full_check(cfg, poison=True, attn_rows=cfg.total_q * cfg.num_q_heads)


MQ_STEP = MQ + [
    # more than 64 query tokens with at most 4 per sequence: the step's own
    # selection in the 4,096-entry kernel, 8 and 16 candidates per lane
    gen.MsaConfig("mq_step_20_seqs", _lens(20, 2_000, 20_000, 5), [4] * 20, 16, 2,
                  permute_pages=True, seed=110),
    gen.MsaConfig("mq_step_20_seqs_100k", [100_000] + _lens(19, 2_000, 9_000, 6), [4] * 20, 16, 2,
                  permute_pages=True, seed=111),
    # the step's own selection with a wavefront selecting two queries of the
    # 7-draft sequence (at most 4 queries per sequence on average)
    gen.MsaConfig("mq_step_skewed", [30_000, 9_000, 5_000, 700], [7, 1, 2, 1], 48, 8,
                  permute_pages=True, seed=107),
    # 513..1024 blocks: 16 candidates per lane in the step's own selection
    gen.MsaConfig("mq_782_blocks", [100_000, 70_000, 3_000], [3, 2, 4], 24, 4, permute_pages=True,
                  seed=106),
    gen.MsaConfig("multi_query_decode", [9000, 20000, 3000, 700], [4, 4, 2, 3], 12, 3,
                  permute_pages=True, seed=48),
]


@pytest.mark.parametrize("cfg", MQ_STEP, ids=lambda c: c.name)
def test_multi_query_step_equals_the_three_calls(cfg):
    """msa_multi_query_step (its own in-kernel selection with at most 4 queries
    per sequence on average, T x k <= 4096 and rows at most 1024 blocks wide,
    else the three calls' launches)
    against msa_index_score -> msa_topk_blocks -> msa_sparse_attn_prefill, bit
    for bit: outputs, log-sum-exps and the selection; run twice."""
    print(f"[mq step] {cfg.name} T={cfg.total_q} maxblk={cfg.max_blocks}", flush=True)
    x = gen.make_inputs(cfg, device="cuda", poison_padding=True)
    ref = MsaStep(x)
    ref.run()
    step = MsaStep(x, multi=True)
    for _ in range(2):
        step.sel.fill_(-7)
        step.out.fill_(0)
        step.run()
        torch.cuda.synchronize()
        assert torch.equal(step.sel, ref.sel)
        assert torch.equal(step.out, ref.out)
        assert torch.equal(step.lse, ref.lse)
