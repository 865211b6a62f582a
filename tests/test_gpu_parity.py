"""HIP path vs the fp64 oracle, through the C ABI (needs an MI355X)."""
import numpy as np
import pytest
import torch

from block_sparse_attention_03_amd import _lib as L
from block_sparse_attention_03_amd import inputs as gen
from block_sparse_attention_03_amd.pipeline import MsaStep

import parity

pytestmark = pytest.mark.gpu


def test_native_library_is_loaded():
    assert L.abi_version() == 1
    import ctypes
    assert isinstance(L.lib(), ctypes.CDLL)


SMALL = [
    # decode: several blocks, ragged last pages, permuted pool, GQA 4
    gen.MsaConfig("decode_ragged_small", [300, 1000, 4500], [1, 1, 1], 12, 3,
                  permute_pages=True, seed=31),
    # decode: one token, exactly one block, one block + 1, dense (k*Bk >= L)
    gen.MsaConfig("decode_edges", [1, 128, 129, 2048, 2049], [1] * 5, 8, 2,
                  permute_pages=True, extra_pages=3, seed=32),
    # G = 1 and G = 16
    gen.MsaConfig("decode_g1", [5000, 700], [1, 1], 4, 4, seed=33),
    gen.MsaConfig("decode_g16", [3000, 9000], [1, 1], 16, 1, permute_pages=True, seed=34),
    # prefill: two sequences, partial first/last blocks, several row tiles
    gen.MsaConfig("prefill_small", [700, 2100], [37, 130], 8, 2, permute_pages=True, seed=35),
    gen.MsaConfig("prefill_one_block", [100], [100], 6, 1, seed=36),
    # mixed: a sequence with no new tokens, one decode token, a prefill chunk
    gen.MsaConfig("mixed_batch", [4000, 900, 3000], [0, 1, 300], 12, 4, permute_pages=True,
                  seed=37),
    # multi-query decode (speculative drafts): a few queries per sequence,
    # scored by the per-block kernel and attended KV-block-major
    gen.MsaConfig("multi_query_decode", [9000, 20000, 3000, 700], [4, 4, 2, 3], 12, 3,
                  permute_pages=True, seed=48),
    # whole sequences new (positions from 0: early queries see fewer than k
    # blocks), G = 1 (buckets of up to 32 queries are small)
    gen.MsaConfig("prefill_from_scratch_g1", [1500, 300, 2600], [1500, 300, 2600], 4, 4,
                  permute_pages=True, seed=59),
    # more than 128 new tokens per sequence on average: the GEMM scoring form,
    # row groups of several sequences' queries, one sequence with none
    gen.MsaConfig("prefill_gemm_mixed", [3000, 900, 5000], [600, 0, 800], 12, 4,
                  permute_pages=True, seed=60),
]


def _random_config(seed: int) -> "gen.MsaConfig":
    """A seeded random shape: batch size, GQA ratio, index heads, ragged
    lengths (sometimes a multiple of 128, sometimes 1) and, for odd seeds,
    several new tokens per sequence (prefill or mixed), even seeds decode."""
    rng = np.random.default_rng(1000 + seed)
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 3, 4, 6, 8, 16]))
    b = int(rng.integers(1, 7))
    lens = []
    for _ in range(b):
        kind = rng.integers(0, 4)
        if kind == 0:
            lens.append(int(128 * rng.integers(1, 40)))
        elif kind == 1:
            lens.append(int(rng.integers(1, 130)))
        else:
            lens.append(int(rng.integers(130, 6000)))
    if seed % 2 == 0:
        n_new = [1] * b
    else:
        n_new = [int(rng.integers(0, min(L, 200) + 1)) for L in lens]
        if sum(n_new) == 0:
            n_new[0] = 1
    hidx = hkv if rng.integers(0, 3) == 0 else 1
    return gen.MsaConfig(f"random_{seed}", lens, n_new, g * hkv, hkv, num_idx_heads=hidx,
                         permute_pages=bool(rng.integers(0, 2)), extra_pages=int(rng.integers(0, 4)),
                         seed=2000 + seed)


@pytest.mark.parametrize("seed", range(24))
def test_random_shapes_against_the_oracle(seed):
    """Seeded random shapes (see _random_config), poisoned padding: scores,
    selection, page table and attention against the oracle; decode shapes
    also through the fused step (equal to the four calls)."""
    cfg = _random_config(seed)
    print(f"[random] {cfg.name}: lens={cfg.seq_lens} n_new={cfg.n_new} "
          f"Hq={cfg.num_q_heads} Hkv={cfg.num_kv_heads} Hidx={cfg.num_idx_heads}", flush=True)
    x, step = parity.full_check(cfg, poison=True)
    if cfg.is_decode:
        fused = MsaStep(x, fused=True)
        fused.run()
        torch.cuda.synchronize()
        assert torch.equal(fused.sel, step.sel)
        assert torch.equal(fused.out, step.out)
        assert torch.equal(fused.lse, step.lse)


def _random_large_config(seed: int) -> "gen.MsaConfig":
    """Larger seeded shapes: 1-8 sequences of 200 to 140,000 tokens
    (log-uniform), H_kv in {1, 2, 4, 8}, G in {1, 2, 4, 6, 8}; one new token
    per sequence, a few drafts, or up to 2,048 new tokens per sequence."""
    rng = np.random.default_rng(7000 + seed)
    b = int(rng.integers(1, 9))
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 6, 8]))
    lens = [int(np.exp(rng.uniform(np.log(200), np.log(140000)))) for _ in range(b)]
    mode = seed % 3
    if mode == 0:
        n_new = [1] * b
    elif mode == 1:
        n_new = [int(rng.integers(1, 9)) for _ in range(b)]
    else:
        n_new = [int(rng.integers(0, min(L, 2048) + 1)) for L in lens]
    n_new = [min(n, L) for n, L in zip(n_new, lens)]
    if sum(n_new) == 0:
        n_new[0] = 1
    hidx = hkv if rng.integers(0, 3) == 0 else 1
    return gen.MsaConfig(f"random_large_{seed}", lens, n_new, g * hkv, hkv, num_idx_heads=hidx,
                         permute_pages=True, extra_pages=int(rng.integers(0, 4)), seed=3000 + seed)


@pytest.mark.parametrize("seed", range(12))
def test_random_large_shapes_against_the_oracle(seed):
    """Seeded larger shapes (see _random_large_config), poisoned padding:
    sampled scores and attention rows and every selection row against the
    oracle; the one-call form (msa_decode_step for decode, else
    msa_multi_query_step) bit-equal to the separate calls."""
    cfg = _random_large_config(seed)
    print(f"[random] {cfg.name}: lens={cfg.seq_lens} n_new={cfg.n_new} "
          f"Hq={cfg.num_q_heads} Hkv={cfg.num_kv_heads} Hidx={cfg.num_idx_heads}", flush=True)
    x, step = parity.full_check(cfg, poison=True, score_rows=2048, attn_rows=1024)
    one = MsaStep(x, fused=True) if cfg.is_decode else MsaStep(x, multi=True)
    one.run()
    torch.cuda.synchronize()
    assert torch.equal(one.sel, step.sel)
    assert torch.equal(one.out, step.out)
    assert torch.equal(one.lse, step.lse)


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_small_cases_poisoned_padding(cfg):
    parity.full_check(cfg, poison=True)


@pytest.mark.parametrize("cfg", SMALL[:1] + SMALL[4:5] + SMALL[8:10], ids=lambda c: c.name)
def test_per_group_index_keys(cfg):
    parity.full_check(cfg.with_idx_heads(cfg.num_kv_heads), poison=True)


def test_tied_scores_pick_lower_blocks():
    """Index keys constant per block make scores tie across blocks; the
    selection must still equal the oracle's on the GPU's own scores."""
    cfg = gen.MsaConfig("ties", [6000, 3000], [1, 4], 8, 2, seed=38)
    x = gen.make_inputs(cfg, device="cuda")
    # every token of a block gets the same key, chosen from 3 values
    rng = np.random.default_rng(0)
    vals = torch.from_numpy(rng.integers(0, 3, size=cfg.num_pages).astype(np.float32)).cuda()
    x.kidx_cache.copy_((vals[:, None, None, None] * 0.5).expand_as(x.kidx_cache).to(torch.bfloat16))
    x.q_idx.fill_(1.0)
    step = MsaStep(x)
    step.run()
    torch.cuda.synchronize()
    parity.check_scores(cfg, x, step)
    sel = parity.check_selection(cfg, x, step)
    assert (sel >= 0).sum() == cfg.total_q * cfg.num_kv_heads * cfg.topk
    parity.check_attention(cfg, x, step)


def test_closed_forms_constant_v_and_zero_q():
    cfg = gen.MsaConfig("closed_forms", [5000, 2600], [1, 1], 8, 2, seed=39)
    x = gen.make_inputs(cfg, device="cuda")
    x.v_cache.fill_(0.75)
    step = MsaStep(x)
    step.run()
    torch.cuda.synchronize()
    assert torch.all(step.out.float() == 0.75)
    # q = 0: every logit is 0, lse = ln(#tokens), out = mean of the attended V
    x.q.zero_()
    step.run()
    torch.cuda.synchronize()
    n_att = step.row_lens.cpu().numpy().astype(np.float64)
    G = cfg.num_q_heads // cfg.num_kv_heads
    want = np.log(np.repeat(n_att, G)).reshape(cfg.num_seqs, cfg.num_q_heads)
    assert np.allclose(step.lse.cpu().numpy(), want, atol=1e-5)


def test_deterministic_and_page_permutation_invariant():
    base = gen.MsaConfig("perm_a", [7000, 3000, 12000], [1, 1, 1], 12, 2, seed=40)
    x = gen.make_inputs(base, device="cuda")
    s1 = MsaStep(x)
    s1.run()
    out1, lse1, sc1 = s1.out.clone(), s1.lse.clone(), s1.scores.clone()
    s1.run()
    torch.cuda.synchronize()
    assert torch.equal(out1, s1.out) and torch.equal(lse1, s1.lse)
    # same logical data, physically permuted pages
    P = base.num_pages
    perm = torch.from_numpy(np.random.default_rng(1).permutation(P)).cuda()
    for name in ("kidx_cache", "k_cache", "v_cache"):
        t = getattr(x, name)
        moved = torch.empty_like(t)
        moved[perm] = t
        setattr(x, name, moved)
    x.block_table = perm.to(torch.int32)[x.block_table.long()].contiguous()
    s2 = MsaStep(x)
    s2.run()
    torch.cuda.synchronize()
    assert torch.equal(sc1, s2.scores)
    assert torch.equal(out1, s2.out) and torch.equal(lse1, s2.lse)


@pytest.mark.parametrize("i", [1, 2, 5])
def test_decode_workloads(i):
    cfg = gen.config(i)
    parity.full_check(cfg, poison=True)


def test_decode_1m_context():
    parity.full_check(gen.config(4))


def _prefill_sweep_rows(cfg, x, step, seed=11):
    """Attention rows (t * H_q + h) of the 8k chunk chosen to cover the
    block-major kernel's structure, not only a random sample: every head of
    every query at a block's first and last position (p mod 128 = 0 or 127),
    every row of the three largest (group, block) buckets (so every 32-row
    tile of them), one row selecting each nonempty (group, block) bucket, and
    random rows up to 16,384 or more."""
    import oracle
    T, Hq, H = cfg.total_q, cfg.num_q_heads, cfg.num_kv_heads
    G = Hq // H
    _, pos_of = oracle.positions(cfg.seq_lens, gen.bits(x.cu_q))
    sel = step.sel.cpu().numpy()  # [T, H, k]
    heads = np.arange(Hq)
    edge_t = np.nonzero((pos_of % cfg.block_size == 0) | (pos_of % cfg.block_size == cfg.block_size - 1))[0]
    rows = [(edge_t[:, None] * Hq + heads[None, :]).ravel()]
    # buckets: (group, block) -> the queries that selected it
    t_idx = np.repeat(np.arange(T), H * cfg.topk)
    g_idx = np.tile(np.repeat(np.arange(H), cfg.topk), T)
    b_idx = sel.reshape(-1)
    keep = b_idx >= 0
    t_idx, g_idx, b_idx = t_idx[keep], g_idx[keep], b_idx[keep]
    key = g_idx.astype(np.int64) * cfg.max_blocks + b_idx
    uniq, first, counts = np.unique(key, return_index=True, return_counts=True)
    for kb in uniq[np.argsort(-counts, kind="stable")[:3]]:
        g = int(kb // cfg.max_blocks)
        ts = t_idx[key == kb]
        rows.append((ts[:, None] * Hq + g * G + np.arange(G)[None, :]).ravel())
    # one row per bucket: its first selecting query, a head of its group
    g_first = (uniq // cfg.max_blocks).astype(np.int64)
    rows.append(t_idx[first] * Hq + g_first * G + (uniq % G))
    got = np.unique(np.concatenate(rows))
    rng = np.random.default_rng(seed)
    extra = rng.choice(T * Hq, size=max(0, 16384 - got.size) + 2048, replace=False)
    return np.unique(np.concatenate([got, extra])), len(uniq)


def test_chunked_prefill_64k():
    """The 8192-token chunk on a 57,344-token prefix: every selection row
    against the oracle's top-k on the GPU's scores; 4,096+ score rows (every
    group of the queries at block edges, the rest random); 16,384+ attention
    rows chosen by _prefill_sweep_rows."""
    import oracle
    cfg = gen.config(3)
    x, step = parity.run_step(cfg)
    T, H = cfg.total_q, cfg.num_kv_heads
    _, pos_of = oracle.positions(cfg.seq_lens, gen.bits(x.cu_q))
    edge_t = np.nonzero((pos_of % cfg.block_size == 0) | (pos_of % cfg.block_size == cfg.block_size - 1))[0]
    edge_rows = (edge_t[:, None] * H + np.arange(H)[None, :]).ravel()
    others = np.setdiff1d(np.arange(T * H), edge_rows)
    score_rows = np.unique(np.concatenate([
        edge_rows, np.random.default_rng(12).choice(others, size=3072, replace=False)]))
    assert score_rows.size >= 4096
    s_err = parity.check_scores(cfg, x, step, rows=score_rows)
    parity.check_selection(cfg, x, step)
    rows, n_buckets = _prefill_sweep_rows(cfg, x, step)
    assert rows.size >= 16384 and n_buckets == H * cfg.max_blocks
    o_err, l_err = parity.check_attention(cfg, x, step, rows=rows)
    print(f"[parity] {cfg.name}: {score_rows.size} score rows (err/bound {s_err:.3g}), "
          f"{rows.size} attention rows over {n_buckets} buckets (out max abs {o_err:.3g}, "
          f"lse max abs {l_err:.3g})", flush=True)


@pytest.mark.parametrize("drafts", [4, 8])
def test_multi_query_decode_60k(drafts):
    """The bench's multi-query workloads at full size (8 x 60k, 4 or 8 draft
    tokens per sequence, padding poisoned): the three calls against the
    oracle (every score row, selection and attention row), and
    msa_multi_query_step bit-equal to them."""
    import dataclasses
    cfg = dataclasses.replace(gen.config(2), name=f"mq_60k_{drafts}drafts", n_new=[drafts] * 8)
    x, step = parity.full_check(cfg, poison=True, attn_rows=cfg.total_q * cfg.num_q_heads)
    multi = MsaStep(x, multi=True)
    multi.run()
    torch.cuda.synchronize()
    assert torch.equal(multi.sel, step.sel)
    assert torch.equal(multi.out, step.out)
    assert torch.equal(multi.lse, step.lse)


def test_paged_decode_60k_per_group_index_keys():
    parity.full_check(gen.config(2).with_idx_heads(8), poison=True)


@pytest.mark.parametrize("prefill", [False, True], ids=["decode", "prefill"])
def test_graph_replay_matches_eager(prefill):
    """The layer-step captured as one HIP graph: every replay, with eager work
    and synchronisation between replays, equals the eager result bit for bit."""
    cfg = (gen.MsaConfig("graph_prefill", [3000, 900], [200, 64], 12, 4, permute_pages=True,
                         seed=41) if prefill else
           gen.MsaConfig("graph_decode", [9000, 700, 4096], [1, 1, 1], 12, 4,
                         permute_pages=True, seed=42))
    x = gen.make_inputs(cfg, device="cuda")
    step = MsaStep(x)
    step.run()
    torch.cuda.synchronize()
    ref_out, ref_lse, ref_sel = step.out.clone(), step.lse.clone(), step.sel.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step.run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step.run()
    torch.cuda.synchronize()
    for i in range(4):
        step.out.zero_()
        step.sel.fill_(-7)
        step.run()  # eager work between replays
        torch.cuda.synchronize()
        step.out.zero_()
        step.sel.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(step.out, ref_out), f"replay {i}: out differs"
        assert torch.equal(step.lse, ref_lse), f"replay {i}: lse differs"
        assert torch.equal(step.sel, ref_sel), f"replay {i}: sel differs"


@pytest.mark.parametrize("cfg", [
    SMALL[0], SMALL[1], SMALL[3],
    gen.MsaConfig("fused_hidx", [7000, 300], [1, 1], 12, 3, num_idx_heads=3, permute_pages=True,
                  seed=43),
    gen.config(2), gen.config(5), gen.config(4),
    # 160 and 320 rows (more page workgroups than the chip holds at once):
    # each page workgroup of the fused step attends two of its row's slots
    gen.MsaConfig("fused_160_rows", [(37 * i * i) % 20000 + 150 for i in range(20)], [1] * 20,
                  16, 8, permute_pages=True, seed=57),
    gen.MsaConfig("fused_320_rows", [(53 * i * i) % 9000 + 2100 for i in range(40)], [1] * 40,
                  32, 8, permute_pages=True, seed=58),
], ids=lambda c: c.name)
def test_fused_decode_step_equals_the_four_calls(cfg):
    """msa_decode_step makes the same selection and the same page products as
    msa_index_score -> msa_topk_blocks -> msa_build_page_table ->
    msa_sparse_attn_decode: out, lse and sel are bit-identical."""
    print(f"[fused] {cfg.name}", flush=True)
    x = gen.make_inputs(cfg, device="cuda", poison_padding=True)
    ref = MsaStep(x)
    ref.run()
    fused = MsaStep(x, fused=True)
    fused.sel.fill_(-7)
    fused.run()
    torch.cuda.synchronize()
    assert torch.equal(fused.sel, ref.sel)
    assert torch.equal(fused.out, ref.out)
    assert torch.equal(fused.lse, ref.lse)
    if cfg.total_q * cfg.num_q_heads <= 4096:
        parity.check_attention(cfg, x, fused)


def test_fused_decode_step_repeats_and_long_rows():
    """msa_decode_step called again and again on one workspace, on short rows
    (one selecting wavefront per page workgroup) and on rows over 1024 blocks
    (four selecting wavefronts): each call equals the four-call result."""
    for cfg in (gen.MsaConfig("step_repeat", [9000, 3000, 700], [1, 1, 1], 12, 3,
                              permute_pages=True, seed=44),
                gen.MsaConfig("step_long_rows", [140000, 9000], [1, 1], 8, 2,
                              permute_pages=True, seed=45)):
        print(f"[fused-repeat] {cfg.name} maxblk={cfg.max_blocks}", flush=True)
        x = gen.make_inputs(cfg, device="cuda", poison_padding=True)
        ref = MsaStep(x)
        ref.run()
        fused = MsaStep(x, fused=True)
        for i in range(5):
            fused.out.zero_()
            fused.run()
            torch.cuda.synchronize()
            assert torch.equal(fused.out, ref.out), f"{cfg.name} call {i}"
            assert torch.equal(fused.lse, ref.lse), f"{cfg.name} call {i}"
            assert torch.equal(fused.sel, ref.sel), f"{cfg.name} call {i}"


@pytest.mark.parametrize("ctx,n_heads", [(60000, (8, 2)), (100000, (8, 2)), (190000, (4, 1)),
                                          (400000, (4, 1)), (700000, (4, 1))],
                         ids=["one_wave_rows", "one_wave_16_per_lane", "four_wave_rows",
                              "eight_wave_rows", "sixteen_wave_rows"])
def test_quantised_scores_tie_at_the_threshold(ctx, n_heads):
    """Scores on 100 levels: a few blocks share each level, so the k-th
    largest score is usually tied while only a few dozen blocks reach the
    lane-maximum prefilter -- ties are resolved inside the compacted survivor
    set.  Selection equals the oracle's on the GPU's scores, and the fused
    step equals the four calls."""
    hq, hkv = n_heads
    cfg = gen.MsaConfig(f"quantised_{ctx}", [ctx, ctx // 3], [1, 1], hq, hkv,
                        permute_pages=True, seed=46)
    print(f"[quantised] {cfg.name} maxblk={cfg.max_blocks}", flush=True)
    x = gen.make_inputs(cfg, device="cuda")
    rng = np.random.default_rng(1)
    # level/8 is exact in bf16 for level < 256; q = 1 makes a score 64 * level / 8
    levels = rng.integers(0, 100, size=(cfg.num_pages, cfg.num_idx_heads)).astype(np.float32)
    vals = torch.from_numpy(levels / 8.0).cuda()
    x.kidx_cache.copy_(vals[:, :, None, None].expand_as(x.kidx_cache).to(torch.bfloat16))
    x.q_idx.fill_(1.0)
    ref = MsaStep(x)
    ref.run()
    torch.cuda.synchronize()
    sel = parity.check_selection(cfg, x, ref)
    assert (sel >= 0).sum() == cfg.total_q * cfg.num_kv_heads * cfg.topk
    fused = MsaStep(x, fused=True)
    fused.run()
    torch.cuda.synchronize()
    assert torch.equal(fused.sel, ref.sel)
    assert torch.equal(fused.out, ref.out)
    assert torch.equal(fused.lse, ref.lse)


def _step_into(step, ws):
    """msa_decode_step on step's inputs, into step's outputs, with workspace ws."""
    x = step.x
    L.msa_decode_step(step.dims, x.q_idx, x.kidx_cache, x.q, x.k_cache, x.v_cache,
                      x.block_table, x.seq_lens, step.out, step.lse, step.sel, ws)


def test_fused_decode_step_shares_a_workspace_across_shapes():
    """One workspace (uninitialised, sized for the largest shape) serves calls
    of different shapes in turn: each call, with its outputs poisoned first,
    equals the four calls."""
    cfgs = [gen.MsaConfig("ws_a", [9000, 3000, 700], [1, 1, 1], 12, 3, permute_pages=True,
                          seed=61),
            gen.MsaConfig("ws_b", [(41 * i * i) % 30000 + 90 for i in range(12)], [1] * 12, 48, 8,
                          permute_pages=True, seed=62),
            gen.MsaConfig("ws_c", [129, 50000], [1, 1], 16, 2, permute_pages=True, seed=63)]
    cases = []
    for cfg in cfgs:
        x = gen.make_inputs(cfg, device="cuda", poison_padding=True)
        ref = MsaStep(x)
        ref.run()
        cases.append((cfg, MsaStep(x, fused=True), ref))
    torch.cuda.synchronize()
    nbytes = max(L.msa_decode_step_workspace_size(c[1].dims) for c in cases)
    ws = torch.empty((nbytes,), dtype=torch.uint8, device="cuda")
    for i, k in enumerate([0, 1, 0, 2, 1, 2, 0]):
        cfg, step, ref = cases[k]
        print(f"[shared-ws] call {i}: {cfg.name}", flush=True)
        step.out.fill_(float("nan"))
        step.lse.fill_(float("nan"))
        step.sel.fill_(-7)
        _step_into(step, ws)
        torch.cuda.synchronize()
        assert torch.equal(step.out, ref.out), f"call {i} ({cfg.name}): out"
        assert torch.equal(step.lse, ref.lse), f"call {i} ({cfg.name}): lse"
        assert torch.equal(step.sel, ref.sel), f"call {i} ({cfg.name}): sel"


def test_prepared_calls_read_current_contents():
    """A PreparedCall passes the same pointers again: after the inputs change
    in place, its result equals a fresh, unprepared call on the new contents
    (and differs from the result before the change)."""
    cfg = gen.MsaConfig("prepared", [9000, 3000, 700], [1, 1, 1], 12, 3, permute_pages=True,
                        seed=65)
    print(f"[prepared] {cfg.name}", flush=True)
    x = gen.make_inputs(cfg, device="cuda", poison_padding=True)
    step = MsaStep(x, fused=True)
    step.run()
    torch.cuda.synchronize()
    before = step.out.clone()
    g = torch.Generator(device="cuda").manual_seed(5)
    x.q.copy_(torch.randn(x.q.shape, generator=g, device="cuda").to(torch.bfloat16))
    x.q_idx.copy_(torch.randn(x.q_idx.shape, generator=g, device="cuda").to(torch.bfloat16))
    step.run()
    fresh = MsaStep(x, fused=True)
    L.msa_decode_step(fresh.dims, x.q_idx, x.kidx_cache, x.q, x.k_cache, x.v_cache,
                      x.block_table, x.seq_lens, fresh.out, fresh.lse, fresh.sel, fresh.workspace)
    torch.cuda.synchronize()
    assert torch.equal(step.out, fresh.out)
    assert torch.equal(step.lse, fresh.lse)
    assert torch.equal(step.sel, fresh.sel)
    assert not torch.equal(step.out, before)


def test_fused_decode_step_rows_past_8192_blocks():
    """Rows of more than 8192 blocks select in the standalone kernel inside
    msa_decode_step; the result still equals the four calls."""
    cfg = gen.MsaConfig("step_8300_blocks", [8300 * 128 - 5, 3000], [1, 1], 2, 1,
                        permute_pages=True, seed=47)
    print(f"[fused-past-8192] maxblk={cfg.max_blocks}", flush=True)
    x = gen.make_inputs(cfg, device="cuda", poison_padding=True)
    ref = MsaStep(x)
    ref.run()
    for with_sel in (True, False):
        fused = MsaStep(x, fused=True)
        fused.sel.fill_(-7)
        L.msa_decode_step(fused.dims, x.q_idx, x.kidx_cache, x.q, x.k_cache, x.v_cache,
                          x.block_table, x.seq_lens, fused.out, fused.lse,
                          fused.sel if with_sel else None, fused.workspace)
        torch.cuda.synchronize()
        if with_sel:
            assert torch.equal(fused.sel, ref.sel)
        assert torch.equal(fused.out, ref.out)
        assert torch.equal(fused.lse, ref.lse)


def _new_rows(cfg, x, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    T = cfg.total_q
    k_new = torch.randn((T, cfg.num_kv_heads, cfg.head_dim), generator=g, device="cuda").to(torch.bfloat16)
    v_new = torch.randn((T, cfg.num_kv_heads, cfg.head_dim), generator=g, device="cuda").to(torch.bfloat16)
    i_new = torch.randn((T, cfg.num_idx_heads, cfg.idx_dim), generator=g, device="cuda").to(torch.bfloat16)
    return k_new, v_new, i_new


@pytest.mark.parametrize("cfg", [SMALL[0], SMALL[6], SMALL[7],
                                 SMALL[1].with_idx_heads(SMALL[1].num_kv_heads)],
                         ids=lambda c: f"{c.name}_hidx{c.num_idx_heads}")
def test_append_kv_matches_the_oracle(cfg):
    """msa_append_kv writes each new token's K, V and index-key rows into its
    page slot and nothing else: the three caches equal the oracle's, bit for
    bit (decode, a mixed batch with a sequence of no new tokens, multi-query
    decode, per-group index keys)."""
    import oracle
    print(f"[append] {cfg.name} Hidx={cfg.num_idx_heads}", flush=True)
    x = gen.make_inputs(cfg, device="cuda")
    k_new, v_new, i_new = _new_rows(cfg, x, 70)
    before = [gen.bits(t) for t in (x.k_cache, x.v_cache, x.kidx_cache)]
    L.msa_append_kv(L.dims_for(cfg), cfg.total_q, k_new, v_new, i_new, x.block_table, x.seq_lens,
                    x.cu_q, x.k_cache, x.v_cache, x.kidx_cache)
    torch.cuda.synchronize()
    ref = oracle.append_kv(*before, gen.bits(k_new), gen.bits(v_new), gen.bits(i_new),
                           gen.bits(x.block_table), gen.bits(x.seq_lens), gen.bits(x.cu_q),
                           cfg.block_size)
    for name, got, want in zip(("k_cache", "v_cache", "kidx_cache"),
                               (x.k_cache, x.v_cache, x.kidx_cache), ref):
        assert np.array_equal(gen.bits(got), want), name


def test_append_then_decode_step_equals_the_full_cache():
    """The decode step after appending the current tokens (their slots
    poisoned first) equals the step on the cache that already held them."""
    import oracle
    cfg = gen.MsaConfig("append_step", [9000, 3000, 700, 128], [1] * 4, 12, 3, permute_pages=True,
                        seed=66)
    print(f"[append-step] {cfg.name}", flush=True)
    x = gen.make_inputs(cfg, device="cuda")
    ref = MsaStep(x, fused=True)
    ref.run()
    torch.cuda.synchronize()
    seq_of, pos_of = oracle.positions(cfg.seq_lens, gen.bits(x.cu_q))
    bt = gen.bits(x.block_table)
    pages = torch.tensor([int(bt[s][p // cfg.block_size]) for s, p in zip(seq_of, pos_of)],
                         device="cuda", dtype=torch.long)
    slots = torch.tensor([int(p % cfg.block_size) for p in pos_of], device="cuda", dtype=torch.long)
    k_new = x.k_cache[pages, :, slots, :].clone()
    v_new = x.v_cache[pages, :, slots, :].clone()
    i_new = x.kidx_cache[pages, :, slots, :].clone()
    nan = float("nan")
    x.k_cache[pages, :, slots, :] = nan
    x.v_cache[pages, :, slots, :] = nan
    x.kidx_cache[pages, :, slots, :] = nan
    L.msa_append_kv(L.dims_for(cfg), cfg.total_q, k_new, v_new, i_new, x.block_table, x.seq_lens,
                    x.cu_q, x.k_cache, x.v_cache, x.kidx_cache)
    step = MsaStep(x, fused=True)
    step.run()
    torch.cuda.synchronize()
    assert torch.equal(step.sel, ref.sel)
    assert torch.equal(step.out, ref.out)
    assert torch.equal(step.lse, ref.lse)


def _check_step_append(cfg, seed):
    """msa_decode_step_append against msa_append_kv + msa_decode_step on copies
    of the same caches, whose new slots are poisoned with NaN first: caches,
    selection, output and LSE equal bit for bit, caches equal to the oracle's
    append."""
    import oracle
    x = gen.make_inputs(cfg, device="cuda")
    k_new, v_new, i_new = _new_rows(cfg, x, seed)
    seq_of, pos_of = oracle.positions(cfg.seq_lens, gen.bits(x.cu_q))
    bt = gen.bits(x.block_table)
    pages = torch.tensor([int(bt[s][p // cfg.block_size]) for s, p in zip(seq_of, pos_of)],
                         device="cuda", dtype=torch.long)
    slots = torch.tensor([int(p % cfg.block_size) for p in pos_of], device="cuda", dtype=torch.long)
    for c in (x.k_cache, x.v_cache, x.kidx_cache):
        c[pages, :, slots, :] = float("nan")
    before = [gen.bits(t) for t in (x.k_cache, x.v_cache, x.kidx_cache)]
    want = oracle.append_kv(*before, gen.bits(k_new), gen.bits(v_new), gen.bits(i_new),
                            bt, cfg.seq_lens, gen.bits(x.cu_q), cfg.block_size)
    del before
    d = L.dims_for(cfg)
    B, Hq, H = cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads

    def outputs():
        ws = torch.empty(L.msa_decode_step_workspace_size(d), dtype=torch.uint8, device="cuda")
        return (torch.empty_like(x.q), torch.empty((B, Hq), dtype=torch.float32, device="cuda"),
                torch.empty((B, H, cfg.topk), dtype=torch.int32, device="cuda"), ws)

    caches_a = [t.clone() for t in (x.k_cache, x.v_cache, x.kidx_cache)]
    out_a, lse_a, sel_a, ws_a = outputs()
    L.msa_append_kv(d, B, k_new, v_new, i_new, x.block_table, x.seq_lens, x.cu_q, *caches_a)
    L.msa_decode_step(d, x.q_idx, caches_a[2], x.q, caches_a[0], caches_a[1], x.block_table,
                      x.seq_lens, out_a, lse_a, sel_a, ws_a)
    out_b, lse_b, sel_b, ws_b = outputs()
    L.msa_decode_step_append(d, k_new, v_new, i_new, x.q_idx, x.kidx_cache, x.q, x.k_cache,
                             x.v_cache, x.block_table, x.seq_lens, out_b, lse_b, sel_b, ws_b)
    torch.cuda.synchronize()
    for name, got_a, got_b, ref in zip(("k", "v", "kidx"), caches_a,
                                       (x.k_cache, x.v_cache, x.kidx_cache), want):
        assert np.array_equal(gen.bits(got_a), ref), name
        assert np.array_equal(gen.bits(got_b), ref), name
    assert torch.equal(sel_b, sel_a)
    assert torch.equal(out_b, out_a)
    assert torch.equal(lse_b, lse_a)
    assert torch.isfinite(lse_b).all()


@pytest.mark.parametrize("hidx", [1, 3])
def test_decode_step_append_equals_append_then_step(hidx):
    """The append inside the decode step's scoring launch
    (msa_decode_step_append) equals msa_append_kv + msa_decode_step.  Lengths
    put the new token at slots 0, 59 and 127 of a block, in the first and in
    later blocks, with one index head and with one per KV group."""
    cfg = gen.MsaConfig("step_append", [9000, 3000, 700, 128, 1, 129], [1] * 6, 12, 3,
                        permute_pages=True, seed=67).with_idx_heads(hidx)
    print(f"[step-append] {cfg.name}", flush=True)
    _check_step_append(cfg, 71)


def test_decode_step_append_rows_past_8192_blocks():
    """The same equality when a row has more than 8192 blocks, so that the step
    selects in the standalone kernels after the appending scoring launch."""
    cfg = gen.MsaConfig("step_append_8300_blocks", [8300 * 128 - 5, 3000], [1, 1], 2, 1,
                        permute_pages=True, seed=48)
    print(f"[step-append-past-8192] maxblk={cfg.max_blocks}", flush=True)
    _check_step_append(cfg, 72)


def test_decode_step_append_at_the_headline_size():
    """The 8 x 60,000 paged decode: msa_decode_step_append against
    msa_append_kv + msa_decode_step, compared on the GPU (caches, selection,
    output and LSE bit for bit; each new slot holds exactly the new rows)."""
    cfg = gen.config(2)
    print(f"[step-append-headline] {cfg.name}", flush=True)
    x = gen.make_inputs(cfg, device="cuda")
    k_new, v_new, i_new = _new_rows(cfg, x, 73)
    d = L.dims_for(cfg)
    B, Hq, H = cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads
    L_s = torch.tensor(cfg.seq_lens, device="cuda", dtype=torch.long) - 1
    pages = x.block_table.long()[torch.arange(B, device="cuda"), L_s // cfg.block_size]
    slots = L_s % cfg.block_size

    def outputs():
        ws = torch.empty(L.msa_decode_step_workspace_size(d), dtype=torch.uint8, device="cuda")
        return (torch.empty_like(x.q), torch.empty((B, Hq), dtype=torch.float32, device="cuda"),
                torch.empty((B, H, cfg.topk), dtype=torch.int32, device="cuda"), ws)

    caches_a = [t.clone() for t in (x.k_cache, x.v_cache, x.kidx_cache)]
    out_a, lse_a, sel_a, ws_a = outputs()
    L.msa_append_kv(d, B, k_new, v_new, i_new, x.block_table, x.seq_lens, x.cu_q, *caches_a)
    L.msa_decode_step(d, x.q_idx, caches_a[2], x.q, caches_a[0], caches_a[1], x.block_table,
                      x.seq_lens, out_a, lse_a, sel_a, ws_a)
    out_b, lse_b, sel_b, ws_b = outputs()
    L.msa_decode_step_append(d, k_new, v_new, i_new, x.q_idx, x.kidx_cache, x.q, x.k_cache,
                             x.v_cache, x.block_table, x.seq_lens, out_b, lse_b, sel_b, ws_b)
    torch.cuda.synchronize()
    for a, b_, new in zip(caches_a, (x.k_cache, x.v_cache, x.kidx_cache), (k_new, v_new, i_new)):
        assert torch.equal(a, b_)
        assert torch.equal(b_[pages, :, slots, :].view(torch.int16), new.view(torch.int16))
    assert torch.equal(sel_b, sel_a)
    assert torch.equal(out_b, out_a)
    assert torch.equal(lse_b, lse_a)


def _dense_decode(cfg, x):
    d = L.dims_for(cfg)
    ws = torch.empty(L.msa_dense_decode_workspace_size(d), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(x.q)
    lse = torch.empty((cfg.num_seqs, cfg.num_q_heads), dtype=torch.float32, device="cuda")
    L.msa_dense_attn_decode(d, x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, out, lse, ws)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("cfg", [SMALL[0], SMALL[1], SMALL[3], gen.config(1)], ids=lambda c: c.name)
def test_dense_decode_baseline_matches_oracle(cfg):
    """The dense GQA baseline attends every cached token: equal to the
    oracle's fixed-page attention over each row's whole block table."""
    import oracle
    print(f"[dense] {cfg.name}", flush=True)
    x = gen.make_inputs(cfg, device="cuda", poison_padding=True)
    out, lse = _dense_decode(cfg, x)
    H = cfg.num_kv_heads
    pt = np.repeat(gen.bits(x.block_table), H, axis=0)
    rl = np.repeat(np.asarray(cfg.seq_lens, dtype=np.int32), H)
    ref_o, ref_l = oracle.paged_attention(gen.bits(x.q), gen.bits(x.k_cache), gen.bits(x.v_cache),
                                          pt, rl)
    got_o = out.float().cpu().numpy()
    assert np.isfinite(got_o).all()
    err = np.abs(got_o - ref_o)
    lim = parity.OUT_ATOL + parity.OUT_RTOL * np.abs(ref_o)
    assert (err <= lim).all(), f"out max abs err {err.max():.3g}"
    assert np.abs(lse.cpu().numpy() - ref_l).max() <= parity.LSE_ATOL


def test_dense_decode_equals_msa_when_every_block_is_selected():
    """With k*Bk >= L every block is selected, so MSA's decode step and the
    dense baseline compute the same attention (different partial splits:
    equal within the output tolerance)."""
    cfg = gen.MsaConfig("dense_vs_msa", [2048, 1500, 700, 130], [1] * 4, 16, 4,
                        permute_pages=True, seed=49)
    x = gen.make_inputs(cfg, device="cuda", poison_padding=True)
    msa = MsaStep(x, fused=True)
    msa.run()
    out, lse = _dense_decode(cfg, x)
    err = (msa.out.float() - out.float()).abs()
    lim = parity.OUT_ATOL + parity.OUT_RTOL * out.float().abs()
    assert bool((err <= lim).all()), f"max abs diff {err.max().item():.3g}"
    assert (msa.lse - lse).abs().max().item() <= parity.LSE_ATOL


def test_decode_at_the_maximum_row_length():
    """A decode row of 16384 blocks (2,097,152 tokens), the largest the ABI
    accepts, next to a short one: full parity through the four calls, and the
    fused step (which routes rows past 8192 blocks through the standalone
    selection) equals them."""
    cfg = gen.MsaConfig("decode_max_blocks", [16384 * 128, 5000], [1, 1], 2, 1,
                        permute_pages=True, seed=50)
    print(f"[max] maxblk={cfg.max_blocks}", flush=True)
    assert cfg.max_blocks == 16384
    x, step = parity.full_check(cfg, poison=True)
    fused = MsaStep(x, fused=True)
    fused.run()
    torch.cuda.synchronize()
    assert torch.equal(fused.sel, step.sel)
    assert torch.equal(fused.out, step.out)
    assert torch.equal(fused.lse, step.lse)


def test_fused_decode_step_graph_replay():
    """msa_decode_step captured as one HIP graph: every replay, with eager work
    and synchronisation between replays, equals the eager result bit for bit."""
    cfg = gen.MsaConfig("graph_fused", [9000, 700, 140000], [1, 1, 1], 12, 4,
                        permute_pages=True, seed=51)
    x = gen.make_inputs(cfg, device="cuda")
    step = MsaStep(x, fused=True)
    step.run()
    torch.cuda.synchronize()
    ref_out, ref_lse, ref_sel = step.out.clone(), step.lse.clone(), step.sel.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step.run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step.run()
    torch.cuda.synchronize()
    for i in range(4):
        step.out.zero_()
        step.sel.fill_(-7)
        step.run()
        torch.cuda.synchronize()
        step.out.zero_()
        step.sel.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(step.out, ref_out), f"replay {i}: out differs"
        assert torch.equal(step.lse, ref_lse), f"replay {i}: lse differs"
        assert torch.equal(step.sel, ref_sel), f"replay {i}: sel differs"


def _dense_prefill(cfg, x):
    d = L.dims_for(cfg)
    out = torch.empty_like(x.q)
    lse = torch.empty((cfg.total_q, cfg.num_q_heads), dtype=torch.float32, device="cuda")
    L.msa_dense_attn_prefill(d, cfg.total_q, x.q, x.k_cache, x.v_cache, x.block_table,
                             x.seq_lens, x.cu_q, out, lse)
    torch.cuda.synchronize()
    return out, lse


def _dense_prefill_oracle(cfg, x, tokens):
    """Each sampled query token as a one-token row over its sequence's block
    table, cut at its own position: dense causal attention by definition."""
    import oracle
    seq_of, pos_of = oracle.positions(cfg.seq_lens, gen.bits(x.cu_q))
    H = cfg.num_kv_heads
    bt = gen.bits(x.block_table)
    pt = np.repeat(bt[seq_of[tokens]], H, axis=0)
    rl = np.repeat(pos_of[tokens] + 1, H).astype(np.int32)
    q = gen.bits(x.q)[tokens]
    return oracle.paged_attention(q, gen.bits(x.k_cache), gen.bits(x.v_cache), pt, rl)


def _check_dense_prefill(cfg, x, out, lse, tokens):
    ref_o, ref_l = _dense_prefill_oracle(cfg, x, tokens)
    got_o = out.float().cpu().numpy()[tokens]
    assert np.isfinite(got_o).all()
    err = np.abs(got_o - ref_o)
    lim = parity.OUT_ATOL + parity.OUT_RTOL * np.abs(ref_o)
    assert (err <= lim).all(), f"out max abs err {err.max():.3g} (worst ratio {(err / lim).max():.3g})"
    assert np.abs(lse.cpu().numpy()[tokens] - ref_l).max() <= parity.LSE_ATOL


@pytest.mark.parametrize("cfg", [SMALL[4], SMALL[5], SMALL[6], SMALL[7],
                                 gen.MsaConfig("dense_prefill_g16", [1000, 3000], [300, 1],
                                               16, 1, permute_pages=True, seed=52)],
                         ids=lambda c: c.name)
def test_dense_prefill_baseline_matches_oracle(cfg):
    """Every query token of the dense causal prefill baseline against the
    oracle's attention over the whole prefix up to the token's position."""
    print(f"[dense prefill] {cfg.name}", flush=True)
    x = gen.make_inputs(cfg, device="cuda", poison_padding=True)
    out, lse = _dense_prefill(cfg, x)
    _check_dense_prefill(cfg, x, out, lse, np.arange(cfg.total_q))


def test_dense_prefill_chunk_on_a_long_prefix_sampled():
    """The 8192-token chunk on a 57,344-token prefix (48 query heads, 8 KV
    heads): 14 sampled query tokens, among them the first and last of the
    chunk, against the oracle."""
    cfg = gen.config(3)
    print(f"[dense prefill] {cfg.name}", flush=True)
    x = gen.make_inputs(cfg, device="cuda", poison_padding=True)
    out, lse = _dense_prefill(cfg, x)
    rng = np.random.default_rng(7)
    tokens = np.unique(np.concatenate([[0, 127, 128, cfg.total_q - 1],
                                       rng.integers(0, cfg.total_q, 10)]))
    _check_dense_prefill(cfg, x, out, lse, tokens)


def test_dense_prefill_equals_msa_when_every_block_is_selected():
    """Contexts of at most 16 blocks: MSA selects every block, so its
    prefill and the dense baseline attend the same tokens."""
    cfg = gen.MsaConfig("dense_vs_msa_prefill", [2048, 1500, 700], [700, 1, 130], 12, 3,
                        permute_pages=True, seed=53)
    x = gen.make_inputs(cfg, device="cuda", poison_padding=True)
    msa = MsaStep(x)
    msa.run()
    out, lse = _dense_prefill(cfg, x)
    err = (msa.out.float() - out.float()).abs()
    lim = parity.OUT_ATOL + parity.OUT_RTOL * out.float().abs()
    assert bool((err <= lim).all()), f"max abs diff {err.max().item():.3g}"
    assert (msa.lse - lse).abs().max().item() <= parity.LSE_ATOL


@pytest.mark.parametrize("cfg", [
    # G = 6: a block chosen by up to 5 drafts is 30 rows (two 16-row
    # passes); the drafts' shared own block holds 5 or 6 queries (36 rows)
    gen.MsaConfig("mq_g6_5drafts", [9000, 20000, 4100], [5, 6, 5], 48, 8, permute_pages=True,
                  seed=54),
    # G = 16: at most 2 queries (32 rows) per small bucket
    gen.MsaConfig("mq_g16_3drafts", [7000, 3000], [3, 2], 16, 1, permute_pages=True, seed=55),
], ids=lambda c: c.name)
def test_small_and_large_buckets(cfg):
    """Few queries per sequence (the multi-query kernel: each (sequence,
    group)'s union of selected blocks, each block attended once for all the
    drafts that chose it, in 16-row passes); every output row against the
    oracle."""
    print(f"[buckets] {cfg.name}", flush=True)
    parity.full_check(cfg, poison=True)


def test_prefill_entry_with_one_query_per_sequence():
    """Single-query sequences through msa_sparse_attn_prefill (every bucket
    small): equal to the oracle, and to the decode path's attention."""
    cfg = gen.MsaConfig("prefill_entry_one_query", [5000, 700, 12000], [1, 1, 1], 12, 4,
                        permute_pages=True, seed=56)
    x = gen.make_inputs(cfg, device="cuda", poison_padding=True)
    step = MsaStep(x, prefill=True)
    step.run()
    torch.cuda.synchronize()
    parity.check_scores(cfg, x, step)
    parity.check_selection(cfg, x, step)
    parity.check_attention(cfg, x, step)
    dec = MsaStep(x)
    dec.run()
    torch.cuda.synchronize()
    assert torch.equal(dec.sel, step.sel)
    err = (dec.out.float() - step.out.float()).abs()
    lim = parity.OUT_ATOL + parity.OUT_RTOL * dec.out.float().abs()
    assert bool((err <= lim).all()), f"max abs diff {err.max().item():.3g}"


def test_validate_inputs_finds_each_fault():
    """msa_validate_inputs: 0 on the generated inputs, and the right bit for a
    length of 0, a length past the block table, a decreasing query range and
    a page index past the pool."""
    cfg = gen.MsaConfig("validate", [3000, 700, 5000], [3, 1, 2], 8, 2, permute_pages=True, seed=60)
    x = gen.make_inputs(cfg, device="cuda")
    d = L.dims_for(cfg)
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")

    def run(bt, sl, cq):
        L.msa_validate_inputs(d, cfg.total_q, bt, sl, cq, status)
        torch.cuda.synchronize()
        return int(status.item())

    assert run(x.block_table, x.seq_lens, x.cu_q) == 0
    assert run(x.block_table, x.seq_lens, None) == 0  # decode-style check, no query ranges
    sl = x.seq_lens.clone()
    sl[1] = 0
    assert run(x.block_table, sl, x.cu_q) & L.MSA_FAULT_SEQ_LEN
    sl = x.seq_lens.clone()
    sl[0] = cfg.max_blocks * cfg.block_size + 1
    assert run(x.block_table, sl, x.cu_q) == L.MSA_FAULT_SEQ_LEN
    cq = x.cu_q.clone()
    cq[2] = cq[1] - 1
    assert run(x.block_table, x.seq_lens, cq) == L.MSA_FAULT_CU_Q
    bt = x.block_table.clone()
    bt[2, 3] = cfg.num_pages
    assert run(bt, x.seq_lens, x.cu_q) == L.MSA_FAULT_BLOCK_TABLE
    bt[0, 0] = -1
    sl = x.seq_lens.clone()
    sl[1] = 0
    assert run(bt, sl, x.cu_q) == L.MSA_FAULT_BLOCK_TABLE | L.MSA_FAULT_SEQ_LEN | L.MSA_FAULT_CU_Q
