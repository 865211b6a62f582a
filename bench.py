#!/usr/bin/env python3
"""Benchmark one MSA layer-step on one MI355X and print ONE JSON line.

Headline workload: paged decode, 8 sequences at a 60,000-token cached prefix,
H_q = 48, H_kv = 8, head_dim 128, idx_dim 64, Bk = 128, k = 16, physical pages
randomly permuted, keys given a per-block scale (seeded synthetic bf16 data).
A step is the whole hot path -- scoring, top-k, page table, sparse attention,
merge -- with inputs resident in HBM.  ``value`` times the fused entry point
msa_decode_step; the four separate calls msa_index_score -> msa_topk_blocks ->
msa_build_page_table -> msa_sparse_attn_decode (bit-identical results) are
timed alongside.

Timing.  The workload is instantiated for several layers, each with its own
K/V and index-key caches (together several times the 256 MB Infinity Cache),
and K layer-steps run back to back cycling over the layers, as a decode pass
over a model does: every step reads its inputs from HBM, and kernels follow
each other with no host or timing gaps.  One pair of HIP events on the
kernels' stream brackets the K steps; ``value`` is their mean.  The roofline
kernel is timed the same way: K back-to-back calls of it over the layers.

Also reported (``also``): decode at 4096 tokens (batch 1), the 60k decode with
one index key per KV group (H_idx = H_kv), ragged decode (16 sequences, 4096 to
524,288 tokens), 1M-context decode (batch 4) with its
scoring pass measured separately, 8192-token chunked prefill onto a
57,344-token prefix (tokens/s), multi-query decode (4 drafts per sequence),
the selection kernel against torch.topk, the dense GQA decode baseline
(msa_dense_attn_decode) at 60k and 1M, and the dense causal prefill baseline
(msa_dense_attn_prefill) on the 8192-token chunk, each with MSA's speedup over
it.  The headline layer-step is also timed as one HIP graph per pass over the
layers.  Roofline fractions are given against the
published peaks and against ceilings measured in the same run
(``measured_ceilings``: a streaming read and a matrix-core loop).  The
oracle's CPU time on the headline workload is reported as ``cpu_baseline``.
"""
from __future__ import annotations

import argparse
import json
import sys
import time

METRIC = "MSA decode µs/layer-step & prefill tok/s at 60k/1M ctx; % HBM/MFMA peak"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--layers", type=int, default=8,
                    help="distinct layers (caches) cycled over by the headline workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-also", action="store_true", help="headline workload only")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="rough CPU budget for the oracle baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run plain 256 MiB device copies (PMC byte-counter calibration)")
    ap.add_argument("--score-only", action="store_true",
                    help="only run the headline's index_score_kernel calls (PMC passes)")
    ap.add_argument("--step-only", action="store_true",
                    help="only run msa_decode_step layer-steps of --config (PMC passes)")
    ap.add_argument("--config", type=int, default=2, choices=(2, 4, 5),
                    help="decode workload of --step-only: 2 = 8 x 60k (headline), 4 = 4 x 1M, "
                         "5 = ragged 16 sequences")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only run chunked-prefill layer-steps, 8192 tokens on 57,344 (PMC passes)")
    ap.add_argument("--gemm-probe", action="store_true",
                    help="only run the bf16 rate probes (constant-operand MFMA loop, vendor GEMM "
                         "8192^3 on N(0,1) and on constant operands) and the 8k chunk's scoring "
                         "GEMM (PMC passes: clocks and matrix-core busy cycles)")
    ap.add_argument("--record-traffic", nargs=5,
                    metavar=("RECORD", "COPY_FETCH", "COPY_WRITE", "FETCH", "WRITE"),
                    help="write traffic record RECORD (index_score: --score-only passes; "
                         "decode_step, decode_step_1m, decode_step_ragged: --step-only "
                         "--config 2, 4, 5 passes) from four rocprofv3 --pmc counter "
                         "CSVs (copy calibration FETCH_SIZE, WRITE_SIZE; the workload's "
                         "FETCH_SIZE, WRITE_SIZE) and exit; needs no GPU")
    return ap.parse_args()


class HipEvent:
    """A timing-only HIP event recorded on torch's current stream (created with
    hipEventDisableSystemFence: no system-scope cache write-back/invalidate)."""
    _hip = None

    @classmethod
    def _lib(cls):
        if cls._hip is None:
            import ctypes
            lib = ctypes.CDLL("libamdhip64.so")
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
            lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = lib
        return cls._hip

    def __init__(self):
        import ctypes
        self.ev = ctypes.c_void_p()
        rc = self._lib().hipEventCreateWithFlags(ctypes.byref(self.ev), 0x20000000)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed: {rc}")

    def record(self):
        import ctypes
        import torch
        rc = self._lib().hipEventRecord(self.ev, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed: {rc}")

    def elapsed_time(self, end: "HipEvent") -> float:
        import ctypes
        ms = ctypes.c_float()
        rc = self._lib().hipEventElapsedTime(ctypes.byref(ms), self.ev, end.ev)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return float(ms.value)

    def __del__(self):
        if self._hip is not None and self.ev:
            self._hip.hipEventDestroy(self.ev)


def time_calls(fns, steps, warmup):
    """Mean ms of `steps` calls cycling over fns, back to back, one event pair.

    The timed region is bracketed by torch.cuda.synchronize() on both sides.
    """
    import torch
    for i in range(warmup):
        fns[i % len(fns)]()
    torch.cuda.synchronize()
    a, b = HipEvent(), HipEvent()
    a.record()
    for i in range(steps):
        fns[i % len(fns)]()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def step_percentiles(fns, steps, warmup):
    """p10 / p50 / p90 of single-call times (µs), cycling over fns: an event
    before each call and one after the last, all on the stream the calls run
    on, back to back (no synchronisation between calls)."""
    import torch
    for i in range(warmup):
        fns[i % len(fns)]()
    torch.cuda.synchronize()
    evs = [HipEvent() for _ in range(steps + 1)]
    for i in range(steps):
        evs[i].record()
        fns[i % len(fns)]()
    evs[steps].record()
    torch.cuda.synchronize()
    t = sorted(evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(steps))
    pick = lambda q: round(t[min(steps - 1, int(q * steps))], 2)  # noqa: E731
    return {"p10": pick(0.1), "p50": pick(0.5), "p90": pick(0.9), "calls": steps}


def parse_max_clock_mhz(rocminfo_text):
    """Max Clock Freq. (MHz) of the first gfx950 agent in rocminfo's output,
    or None."""
    for agent in rocminfo_text.split("*******"):
        if "gfx950" not in agent or "Max Clock Freq. (MHz):" not in agent:
            continue
        try:
            return int(agent.split("Max Clock Freq. (MHz):")[1].split()[0])
        except (IndexError, ValueError):
            return None
    return None


def gpu_max_clock_mhz():
    """The GPU agent's maximum engine clock as rocminfo reports it, or None."""
    import subprocess
    try:
        txt = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except (OSError, subprocess.SubprocessError):
        return None
    return parse_max_clock_mhz(txt)


def dense_calls(xs):
    """msa_dense_attn_decode (the dense GQA baseline) on each layer's inputs,
    with its buffers allocated once."""
    import torch
    from block_sparse_attention_03_amd import _lib
    fns = []
    for x in xs:
        d = _lib.dims_for(x.cfg)
        ws = torch.empty(_lib.msa_dense_decode_workspace_size(d), dtype=torch.uint8, device="cuda")
        out = torch.empty_like(x.q)
        lse = torch.empty(x.q.shape[:2], dtype=torch.float32, device="cuda")
        fns.append(lambda x=x, d=d, ws=ws, out=out, lse=lse: _lib.msa_dense_attn_decode(
            d, x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, out, lse, ws))
    return fns


def dense_line(cfg, xs, n, msa_ms):
    from block_sparse_attention_03_amd import accounting as acc
    ms = time_calls(dense_calls(xs), n, 2)
    nbytes = sum(cfg.seq_lens) * cfg.num_kv_heads * 4 * cfg.head_dim  # K and V, bf16
    return {"us_per_layer_step": round(ms * 1e3, 2),
            "kv_bytes": int(nbytes),
            "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / acc.HBM_PEAK_GBS, 4),
            "msa_speedup": round(ms / msa_ms, 2)}


def topk_vs_torch(steps_, n):
    """Selection kernel (msa_topk_blocks) against torch.topk(k=16, unsorted) on
    the same block scores, back-to-back calls over the layers.  torch.topk does
    not apply the method's rule (own block forced in, lower-index ties,
    ascending output): this is a speed comparison only."""
    import torch
    for st in steps_:
        st.score()
    torch.cuda.synchronize()
    k = steps_[0].cfg.topk
    ours = time_calls([st.topk for st in steps_], n, 2)
    theirs = time_calls([lambda st=st: torch.topk(st.scores, k, dim=-1, sorted=False)
                         for st in steps_], n, 2)
    rows = steps_[0].scores.shape[0] * steps_[0].scores.shape[1]
    return {"rows": rows, "candidates_per_row": steps_[0].scores.shape[2],
            "msa_topk_blocks_us": round(ours * 1e3, 2), "torch_topk_us": round(theirs * 1e3, 2)}


def append_line(cfg, xs, n, steps_=None):
    """msa_append_kv (the new tokens' K, V and index keys into their pages) on
    each layer's caches, back-to-back calls: µs per call and the bytes it
    moves (each row read once and written once).  With the layers' fused decode
    steps (decode only), also the serving-loop pair -- msa_append_kv then
    msa_decode_step -- against msa_decode_step_append, which appends inside
    the step's scoring launch: µs per layer-step."""
    import torch
    from block_sparse_attention_03_amd import _lib
    g = torch.Generator(device="cuda").manual_seed(5)
    T = cfg.total_q

    def rows(h, dim):
        return torch.randn((T, h, dim), generator=g, device="cuda").to(torch.bfloat16)

    new = [(rows(cfg.num_kv_heads, cfg.head_dim), rows(cfg.num_kv_heads, cfg.head_dim),
            rows(cfg.num_idx_heads, cfg.idx_dim)) for _ in xs]
    calls = [_lib.prepare_msa_append_kv(_lib.dims_for(cfg), T, k, v, i, x.block_table, x.seq_lens,
                                        x.cu_q, x.k_cache, x.v_cache, x.kidx_cache)
             for x, (k, v, i) in zip(xs, new)]
    ms = time_calls(calls, n, 4)
    nbytes = 2 * T * (2 * cfg.num_kv_heads * cfg.head_dim + cfg.num_idx_heads * cfg.idx_dim) * 2
    line = {"us": round(ms * 1e3, 2), "bytes_moved": nbytes,
            "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1)}
    if steps_ is not None and cfg.is_decode:
        pairs = []
        for c, st in zip(calls, steps_):
            pairs += [c, st.fused_step]
        line["append_then_step_us"] = round(time_calls(pairs, 2 * n, 8) * 2e3, 2)
        joint = [_lib.prepare_msa_decode_step_append(
                     st.dims, k, v, i, st.x.q_idx, st.x.kidx_cache, st.x.q, st.x.k_cache,
                     st.x.v_cache, st.x.block_table, st.x.seq_lens, st.out, st.lse, st.sel,
                     st.workspace)
                 for st, (k, v, i) in zip(steps_, new)]
        line["step_append_us"] = round(time_calls(joint, n, 4) * 1e3, 2)
    return line


def time_graph(steps_, steps, warmup):
    """Mean ms per layer-step when the layer-steps of all layers are captured as
    one HIP graph and the graph is replayed back to back."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for st in steps_:
            st.run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for st in steps_:
            st.run()
    reps = max(1, steps // len(steps_))
    ms = time_calls([g.replay], reps, max(1, warmup // len(steps_)))
    del g
    return ms / len(steps_)


def make_layers(cfg, n, device="cuda"):
    """n independent instances of the workload (layer l draws with seed + 1000*l)."""
    import dataclasses
    from block_sparse_attention_03_amd import inputs as gen
    return [gen.make_inputs(dataclasses.replace(cfg, seed=cfg.seed + 1000 * l), device=device)
            for l in range(n)]


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _host(x, names):
    from block_sparse_attention_03_amd import inputs as gen
    return {k: gen.bits(getattr(x, k)) for k in names}


def _selected_pages(x, sel, seq_of):
    """Host copies of the K/V pages a selection touches, and a block table
    mapping each selected (sequence, block) to its row in them (others -> 0):
    the oracle's attention then reads only those pages from host memory."""
    import numpy as np
    import torch
    from block_sparse_attention_03_amd import inputs as gen
    bt = gen.bits(x.block_table)
    T = sel.shape[0]
    pairs = np.unique(np.stack([np.repeat(seq_of[:T], sel.shape[1] * sel.shape[2]),
                                sel.reshape(-1)], axis=1), axis=0)
    pairs = pairs[pairs[:, 1] >= 0]
    pages = torch.from_numpy(bt[pairs[:, 0], pairs[:, 1]].astype(np.int64)).to(x.k_cache.device)
    kp = gen.bits(x.k_cache.index_select(0, pages))
    vp = gen.bits(x.v_cache.index_select(0, pages))
    bt2 = np.zeros_like(bt)
    bt2[pairs[:, 0], pairs[:, 1]] = np.arange(len(pairs), dtype=np.int32)
    return kp, vp, bt2


def cpu_stages(cfg, x, sample_queries=None):
    """Wall seconds of the oracle's stages on one layer-step of `cfg` (inputs
    `x`, already drawn on the GPU): scoring, top-k, page table (decode) and
    attention.  sample_queries: score, select and attend only that many query
    tokens of each sequence, evenly spaced over its new tokens, and scale the
    stage times to the whole step by the query count.  Host copies are not
    timed."""
    import numpy as np
    import oracle
    h = _host(x, ("q_idx", "kidx_cache", "q", "block_table", "seq_lens", "cu_q"))
    H, Hq, k = cfg.num_kv_heads, cfg.num_q_heads, cfg.topk
    seq_of, pos_of = oracle.positions(h["seq_lens"], h["cu_q"])
    T = cfg.total_q
    # a sample: sample_queries query tokens of each sequence, evenly spaced
    # over its query range (so their positions span the chunk's)
    toks = np.arange(T) if sample_queries is None else np.unique(np.concatenate(
        [a + (np.arange(min(sample_queries, b - a)) * (b - a)) // max(1, min(sample_queries, b - a))
         for a, b in zip(h["cu_q"][:-1].astype(np.int64), h["cu_q"][1:].astype(np.int64))]))
    n = len(toks)
    score_rows = (toks[:, None] * H + np.arange(H)[None, :]).ravel()
    t0 = time.perf_counter()
    sc = oracle.index_score(h["q_idx"], h["kidx_cache"], h["block_table"], seq_of, pos_of,
                            cfg.block_size, rows=score_rows)
    t1 = time.perf_counter()
    bl = oracle.b_loc_rows(pos_of, H, cfg.block_size)[score_rows]
    chosen = oracle.topk(sc, bl, k)
    t2 = time.perf_counter()
    sel = np.full((T, H, k), -1, np.int32)
    sel[toks] = chosen.reshape(n, H, k)
    pt_s = 0.0
    if cfg.is_decode and sample_queries is None:
        t3 = time.perf_counter()
        oracle.page_table(sel, h["block_table"], h["seq_lens"], cfg.block_size)
        pt_s = time.perf_counter() - t3
    kp, vp, bt2 = _selected_pages(x, sel, seq_of)
    attn_rows = (toks[:, None] * Hq + np.arange(Hq)[None, :]).ravel()
    t4 = time.perf_counter()
    oracle.attention(h["q"], kp, vp, bt2, seq_of, pos_of, sel, rows=attn_rows)
    t5 = time.perf_counter()
    f = T / n
    st = {"score": (t1 - t0) * f, "topk": (t2 - t1) * f, "page_table": pt_s * f,
          "attention": (t5 - t4) * f}
    out = {"step_s": round(sum(st.values()), 4),
           "stage_s": {a: round(b, 5) for a, b in st.items()},
           "sample": "the whole layer-step" if n == T else
                     f"{n} of {T} query tokens ({sample_queries} per sequence, evenly spaced "
                     f"over its new tokens), stage times scaled by {T}/{n}"}
    return out


def cpu_baseline(cfg, x, budget_s):
    """The oracle (as it stands) on the same decode workload, full layer-steps,
    repeated for about budget_s seconds."""
    import oracle
    h = _host(x, ("q_idx", "kidx_cache", "q", "k_cache", "v_cache", "block_table", "seq_lens",
                  "cu_q"))
    oracle.build(force=False)
    H = cfg.num_kv_heads

    def one_step():
        seq_of, pos_of = oracle.positions(h["seq_lens"], h["cu_q"])
        sc = oracle.index_score(h["q_idx"], h["kidx_cache"], h["block_table"], seq_of,
                                pos_of, cfg.block_size)
        sel = oracle.topk(sc, oracle.b_loc_rows(pos_of, H, cfg.block_size), cfg.topk)
        sel = sel.reshape(cfg.total_q, H, cfg.topk)
        oracle.page_table(sel, h["block_table"], h["seq_lens"], cfg.block_size)
        oracle.attention(h["q"], h["k_cache"], h["v_cache"], h["block_table"],
                         seq_of, pos_of, sel)

    n, t0 = 0, time.perf_counter()
    while True:
        one_step()
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 5000:
            break
    return {"value": round(el * 1e6 / n, 1), "unit": "us/layer-step", "cores": oracle.threads(),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{n} full layer-steps of the headline workload (64 rows scored over "
                      f"60,000 tokens each, top-k, page table, attention), fp64 C with OpenMP, "
                      f"{el:.1f} s",
            "stages": cpu_stages(cfg, x)}


# Traffic records: HBM bytes per launch (per layer-step for the decode step)
# from rocprofv3 FETCH_SIZE / WRITE_SIZE passes, keyed by the SHA-256 of the
# sources the kernels are built from, so that a later change voids them.
CSRC = "block_sparse_attention_03_amd/csrc"
_STEP_SOURCES = ["index_score.hip", "decode_attn.hip", "select.hpp", "decode_tile.hpp",
                 "msa_common.hpp"]
TRAFFIC = {
    "index_score": {
        "file": "profiles/index_score_decode_60k_traffic.json",
        "config": 2,
        "sources": ["index_score.hip"],
        "kernels": ["index_score_kernel<true, false>"],
        "what": "index_score_kernel (the msa_index_score form) per launch",
    },
    "decode_step": {
        "file": "profiles/decode_step_60k_traffic.json",
        "config": 2,
        "sources": _STEP_SOURCES,
        "kernels": ["index_score_kernel<false, false>", "decode_fused_kernel<8, 1, true>",
                    "decode_merge_kernel"],
        "what": "msa_decode_step's three kernels, summed per layer-step",
    },
    "decode_step_1m": {
        "file": "profiles/decode_step_1m_traffic.json",
        "config": 4,
        "sources": _STEP_SOURCES,
        "kernels": ["index_score_kernel<false, false>", "decode_fused_kernel<32, 4, false>",
                    "decode_merge_kernel"],
        "what": "msa_decode_step's three kernels, summed per layer-step",
    },
    "decode_step_ragged": {
        "file": "profiles/decode_step_ragged_traffic.json",
        "config": 5,
        "sources": _STEP_SOURCES,
        "kernels": ["index_score_kernel<false, false>", "decode_multi_kernel<16, 4, true, 4>",
                    "decode_merge_kernel"],
        "what": "msa_decode_step's three kernels, summed per layer-step",
    },
}


def _root():
    import os
    return os.path.dirname(os.path.abspath(__file__))


def sources_sha256(srcs):
    """SHA-256 over the bytes of the source files, in order."""
    import hashlib
    h = hashlib.sha256()
    for path in srcs:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(name):
    """HBM bytes per launch (per layer-step for decode_step) from the traffic
    record `name`, or None if a source has changed since it was taken."""
    import os
    spec = TRAFFIC[name]
    path = os.path.join(_root(), spec["file"])
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    srcs = [os.path.join(_root(), CSRC, f) for f in spec["sources"]]
    if rec.get("source_sha256") != sources_sha256(srcs):
        return None
    return int(rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"])


def traffic_record(name, copy_f, copy_w, fetch, write, srcs):
    """Traffic record `name` from rocprofv3 --pmc counter CSVs: for each of the
    record's kernels, the mean FETCH_SIZE and WRITE_SIZE (KiB) over its
    launches, each scaled by what the same counter reads for a plain 256 MiB
    device copy; the record's totals sum its kernels (one launch each per
    layer-step); `srcs` are hashed into the record."""
    import csv
    from block_sparse_attention_03_amd import accounting as acc
    from block_sparse_attention_03_amd import inputs as gen
    spec = TRAFFIC[name]

    def mean(path, counter, match):
        vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(path))
                if r["Counter_Name"] == counter and match(r["Kernel_Name"])]
        if not vals:
            raise SystemExit(f"{path}: no {counter} rows for the kernel")
        return sum(vals) / len(vals), len(vals)

    copy_bytes = 256 << 20
    is_copy = lambda k: k == "__amd_rocclr_copyBuffer"  # noqa: E731
    cf, _ = mean(copy_f, "FETCH_SIZE", is_copy)
    cw, _ = mean(copy_w, "WRITE_SIZE", is_copy)
    ff, fw = copy_bytes / 1024 / cf, copy_bytes / 1024 / cw
    kernels = []
    for kname in spec["kernels"]:
        kf, nf = mean(fetch, "FETCH_SIZE", lambda k, kn=kname: kn in k)
        kw, nw = mean(write, "WRITE_SIZE", lambda k, kn=kname: kn in k)
        kernels.append({"kernel": kname, "launches": {"fetch_pass": nf, "write_pass": nw},
                        "fetch_size_kib_per_launch": round(kf, 1),
                        "write_size_kib_per_launch": round(kw, 1),
                        "fetch_bytes_per_launch": int(round(kf * 1024 * ff)),
                        "write_bytes_per_launch": int(round(kw * 1024 * fw))})
    cfg = gen.config(spec["config"])
    algo = acc.score_bytes(cfg) + (acc.decode_attn_bytes(cfg) if name.startswith("decode_step") else 0)
    lens = (f"{cfg.seq_lens[0]:,} tokens" if len(set(cfg.seq_lens)) == 1
            else f"{min(cfg.seq_lens):,} to {max(cfg.seq_lens):,} tokens")
    return {
        "record": name,
        "what": spec["what"],
        "workload": f"paged decode ({cfg.name}), {cfg.num_seqs} sequences x {lens}, "
                    f"H_kv {cfg.num_kv_heads}, H_idx {cfg.num_idx_heads}",
        "source_sha256": sources_sha256(srcs),
        "sources": [f"{CSRC}/{f}" for f in spec["sources"]],
        "kernels": kernels,
        "copy_calibration": {"bytes_per_launch": copy_bytes, "fetch_size_kib": round(cf, 1),
                             "write_size_kib": round(cw, 1), "fetch_factor": round(ff, 4),
                             "write_factor": round(fw, 4)},
        "fetch_bytes_per_launch": sum(k["fetch_bytes_per_launch"] for k in kernels),
        "write_bytes_per_launch": sum(k["write_bytes_per_launch"] for k in kernels),
        "algorithmic_bytes_per_launch": algo,
    }


def record_traffic(name, copy_f, copy_w, fetch, write):
    """Write traffic record `name` from the four counter CSVs (see traffic_record)."""
    import os
    if name not in TRAFFIC:
        raise SystemExit(f"unknown traffic record {name!r}: one of {sorted(TRAFFIC)}")
    srcs = [os.path.join(_root(), CSRC, f) for f in TRAFFIC[name]["sources"]]
    rec = traffic_record(name, copy_f, copy_w, fetch, write, srcs)
    with open(os.path.join(_root(), TRAFFIC[name]["file"]), "w") as f:
        json.dump(rec, f, indent=2)
        f.write("\n")
    print(json.dumps(rec))


def measured_ceilings(chain=None):
    """Sustained HBM read bandwidth and bf16 matrix-core rate on this GPU, from
    the separate calibration library: the best over grid-stride and
    chunk-per-workgroup forms of a 2 GiB streaming read; the same for 64 MiB
    reads (the size of one decode layer-step's two passes) cycling over 32
    distinct slices; device copies of 800 and 96 MiB; and independent
    32x32x16 products at 4 and 8 waves per SIMD.  With chain = (a, b, c)
    bytes, also the time of three dependent contiguous reads of a, b and c
    bytes, one launch each, back to back over distinct slices: the floor of
    a three-launch decode step that streams those bytes."""
    import ctypes
    import os
    import torch
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "block_sparse_attention_03_amd",
                        "libmsa_calib.so")
    c = ctypes.CDLL(path)
    c.msa_calib_read_grid.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                      ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    c.msa_calib_read_sink_len.restype = ctypes.c_size_t
    c.msa_calib_copy_grid.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                      ctypes.c_int, ctypes.c_void_p]
    c.msa_calib_read_chunked.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_size_t,
                                         ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    c.msa_calib_copy_chunked.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                         ctypes.c_size_t, ctypes.c_void_p]
    c.msa_calib_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    c.msa_calib_mfma_flop.restype = ctypes.c_double
    c.msa_calib_mfma_flop.argtypes = [ctypes.c_int, ctypes.c_int]
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    nbytes = 2 << 30
    small = 64 << 20
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.empty(c.msa_calib_read_sink_len(), dtype=torch.int32, device="cuda")
    iters = 16384
    out = torch.empty(2048 * 256, dtype=torch.float32, device="cuda")

    # two forms of each: grid-stride loops over a fixed grid ("grid", workgroups)
    # and one short-lived workgroup per contiguous chunk ("chunk", KiB)
    forms = [("grid", g) for g in (256, 512, 1024, 4096)] + [("chunk", k) for k in (16, 32, 64)]

    def read(ptr, size, form):
        kind, v = form
        if kind == "grid":
            rc = c.msa_calib_read_grid(ptr, size, v, sink.data_ptr(), sink.numel(), st)
        else:
            rc = c.msa_calib_read_chunked(ptr, size, v << 10, sink.data_ptr(), sink.numel(), st)
        if rc != 0:
            raise RuntimeError("msa_calib_read failed")

    def copy_bytes(src, dst, size, form):
        kind, v = form
        if kind == "grid":
            rc = c.msa_calib_copy_grid(src, dst, size, v, st)
        else:
            rc = c.msa_calib_copy_chunked(src, dst, size, v << 10, st)
        if rc != 0:
            raise RuntimeError("msa_calib_copy failed")

    def name(form):
        return f"{form[1]} workgroups grid-stride" if form[0] == "grid" else f"{form[1]} KiB per workgroup"

    def mfma(blocks):
        if c.msa_calib_mfma(out.data_ptr(), blocks, iters, st) != 0:
            raise RuntimeError("msa_calib_mfma failed")

    big, sized = {}, {}
    base = buf.data_ptr()
    for form in forms:
        ms = time_calls([lambda f=form: read(base, nbytes, f)], 6, 2)
        big[form] = nbytes / (ms * 1e-3) / 1e9
        fns = [lambda i=i, f=form: read(base + i * small, small, f) for i in range(nbytes // small)]
        ms = time_calls(fns, 2 * len(fns), len(fns))
        sized[form] = small / (ms * 1e-3) / 1e9
    # a device copy of 800 MiB (1.6 GiB of traffic, half reads and half
    # writes: the mix and size of the prefill block-major kernel's traffic)
    half = 800 << 20
    copy = {}
    for form in forms:
        ms = time_calls([lambda f=form: copy_bytes(base, base + half, half, f)], 6, 2)
        copy[form] = 2 * half / (ms * 1e-3) / 1e9
    # the same copy of 96 MiB each way, a footprint the 256 MB Infinity Cache
    # holds: what keeping a round trip's data in that cache could gain
    small_half = 96 << 20
    copy_small = {}
    for form in forms:
        ms = time_calls([lambda f=form: copy_bytes(base, base + small_half, small_half, f)], 40, 8)
        copy_small[form] = 2 * small_half / (ms * 1e-3) / 1e9
    chain_us = None
    if chain:
        # each read in the form fastest at 64 MiB, or one 16 KiB chunk per
        # workgroup for the small one
        sizes = [int(n) // 16 * 16 for n in chain]
        span = sum(sizes)
        best_small = max(sized, key=sized.get)
        kinds = [best_small if n > small // 4 else ("chunk", 16) for n in sizes]

        def chain_call(i):
            off = base + i * span
            for n, f in zip(sizes, kinds):
                read(off, n, f)
                off += n
        fns = [lambda i=i: chain_call(i) for i in range(nbytes // span)]
        chain_us = time_calls(fns, 4 * len(fns), len(fns)) * 1e3
    tflops = {}
    for blocks in (1024, 2048):
        # enough warm-up launches (about 1 ms each) for the clocks to settle
        ms = time_calls([lambda b=blocks: mfma(b)], 10, 5)
        tflops[blocks] = c.msa_calib_mfma_flop(blocks, iters) / (ms * 1e-3) / 1e12
    del buf
    torch.cuda.empty_cache()
    vendor = vendor_gemm_tflops()
    clock = gpu_max_clock_mhz()
    gb, gs, bm = max(big, key=big.get), max(sized, key=sized.get), max(tflops, key=tflops.get)
    gc = max(copy, key=copy.get)
    gcs = max(copy_small, key=copy_small.get)
    res = {"hbm_read_gbs": round(big[gb], 1),
           "hbm_read_64mib_gbs": round(sized[gs], 1),
           "hbm_copy_800mib_gbs": round(copy[gc], 1),
           "copy_96mib_gbs": round(copy_small[gcs], 1),
           "mfma_bf16_tflops": round(tflops[bm], 1),
           "vendor_gemm_bf16_randn_tflops": round(vendor["randn"], 1),
           "vendor_gemm_bf16_const_tflops": round(vendor["const"], 1),
           "gpu_max_clock_mhz": clock,
           "how": f"non-temporal streaming read of 2 GiB (best: {name(gb)}) "
                  f"and of 64 MiB slices back to back (best: {name(gs)}); a device copy of 800 MiB "
                  f"(read + write bytes, best: {name(gc)}) and of 96 MiB (best: {name(gcs)}), "
                  f"each the fastest of grid-stride loops over 256-4096 workgroups of 256 threads "
                  f"and one workgroup per 16, 32 or 64 KiB chunk; 32x32x16 bf16 MFMA "
                  f"loop on constant operands, 4 independent chains per wave, {bm // 256 * 4} waves "
                  f"per CU; torch.matmul (hipBLASLt) bf16 8192^3 on N(0,1) and on all-ones operands",
           "read_gbs_by_form": {name(k): round(v, 1) for k, v in big.items()},
           "read_64mib_gbs_by_form": {name(k): round(v, 1) for k, v in sized.items()},
           "copy_800mib_gbs_by_form": {name(k): round(v, 1) for k, v in copy.items()}}
    if chain_us is not None:
        res["three_read_launches_us"] = round(chain_us, 2)
        res["three_read_launches_bytes"] = [int(n) for n in chain]
    return res


def vendor_gemm_tflops():
    """bf16 rate of the vendor library's GEMM (torch.matmul, hipBLASLt) at
    8192^3, on N(0,1) operands and on all-ones operands.  The matrix cores'
    clock drops under random data, which the constant-operand loop does not
    show: the random-operand rate is what a GEMM on this data can sustain."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    out = {}
    for kind in ("randn", "const"):
        if kind == "randn":
            a = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16, generator=g)
            b = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16, generator=g)
        else:
            a = torch.ones(8192, 8192, device="cuda", dtype=torch.bfloat16)
            b = torch.ones(8192, 8192, device="cuda", dtype=torch.bfloat16)
        c = torch.empty(8192, 8192, device="cuda", dtype=torch.bfloat16)
        ms = time_calls([lambda: torch.matmul(a, b, out=c)], 10, 5)
        out[kind] = 2 * 8192 ** 3 / (ms * 1e-3) / 1e12
        del a, b, c
    torch.cuda.empty_cache()
    return out


def roofline_entry(name, nbytes, ms, traffic=None):
    from block_sparse_attention_03_amd.accounting import HBM_PEAK_GBS
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "kernel": name, "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
            "algorithmic_bytes": int(nbytes), "avg_ms": round(ms, 5)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the library has no "
              f"multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    if args.record_traffic:
        record_traffic(*args.record_traffic)
        return
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    from block_sparse_attention_03_amd import _lib, accounting as acc
    from block_sparse_attention_03_amd import inputs as gen
    from block_sparse_attention_03_amd.pipeline import MsaStep
    _lib.lib()  # fail loudly if the HIP library is missing

    if args.copy_calibration:
        # a plain copy of known size: each launch fetches and writes 256 MiB
        a = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(4):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": a.numel() * 4, "launches": 4}))
        return
    if args.gemm_probe:
        ceil = measured_ceilings()
        cfg = gen.config(3)
        st3 = [MsaStep(x) for x in make_layers(cfg, 2)]
        ms = time_calls([s_.score for s_ in st3], args.steps, args.warmup)
        print(json.dumps({"index_score_gemm_ms": ms,
                          "index_score_gemm_tflops": acc.score_flops(cfg) / (ms * 1e-3) / 1e12,
                          "mfma_bf16_tflops": ceil["mfma_bf16_tflops"],
                          "vendor_gemm_bf16_randn_tflops": ceil["vendor_gemm_bf16_randn_tflops"],
                          "vendor_gemm_bf16_const_tflops": ceil["vendor_gemm_bf16_const_tflops"]}))
        return
    if args.prefill_only:
        cfg = gen.config(3)
        st3 = [MsaStep(x) for x in make_layers(cfg, 2)]
        ms = time_calls([s_.run for s_ in st3], args.steps, args.warmup)
        print(json.dumps({"prefill_step_ms": ms, "launches": args.steps + args.warmup}))
        return
    if args.score_only:
        cfg = gen.config(2)
        four = [MsaStep(x) for x in make_layers(cfg, args.layers)]
        ms = time_calls([s_.score for s_ in four], args.steps, args.warmup)
        print(json.dumps({"index_score_ms": ms, "launches": args.steps + args.warmup}))
        return
    if args.step_only:
        cfg = gen.config(args.config)
        n_layers = args.layers if args.config == 2 else 2  # 18 GB per 1M layer
        fused = [MsaStep(x, fused=True) for x in make_layers(cfg, n_layers)]
        ms = time_calls([s_.run for s_ in fused], args.steps, args.warmup)
        print(json.dumps({"decode_step_ms": ms, "layer_steps": args.steps + args.warmup}))
        return

    # ---------------- headline: paged decode at 60k, batch 8 ----------------
    cfg = gen.config(2)
    layers = make_layers(cfg, args.layers)
    fused = [MsaStep(x, fused=True) for x in layers]   # msa_decode_step
    four = [MsaStep(x) for x in layers]                # the four ABI calls
    fused_ms = time_calls([s.run for s in fused], args.steps, args.warmup)
    four_ms = time_calls([s.run for s in four], args.steps, args.warmup)
    graph_ms = time_graph(fused, args.steps, args.warmup)
    per_step = step_percentiles([s.run for s in fused], args.steps, args.warmup)
    # the scoring pass alone (msa_index_score: the same index_score_kernel)
    score_ms = time_calls([s.score for s in four], args.steps, args.warmup)
    attn_ms = time_calls([s.attend for s in four], args.steps, args.warmup)
    topk_line = {cfg.name: topk_vs_torch(four, args.steps)}
    dense = {cfg.name: dense_line(cfg, layers, max(16, args.steps // 8), fused_ms)}
    layer_bytes = acc.score_bytes(cfg) + acc.decode_attn_bytes(cfg)

    def frac(ms_):
        return round(layer_bytes / (ms_ * 1e-3) / 1e9 / acc.HBM_PEAK_GBS, 4)

    result = {
        "metric": METRIC,
        "value": round(fused_ms * 1e3, 2),
        "unit": "us/layer-step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(fused_ms, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "num_seqs": cfg.num_seqs, "context": cfg.seq_lens[0],
                   "num_q_heads": cfg.num_q_heads, "num_kv_heads": cfg.num_kv_heads,
                   "num_idx_heads": cfg.num_idx_heads, "head_dim": cfg.head_dim,
                   "idx_dim": cfg.idx_dim, "block_size": cfg.block_size, "topk": cfg.topk,
                   "seed": cfg.seed, "layers": args.layers,
                   "timing": "layer-steps back to back over distinct per-layer caches (cold HBM)",
                   "entry_point": "msa_decode_step"},
        # the timed step is msa_decode_step's three kernels, one launch each;
        # the select-and-attend kernel is the longest of them (kernel trace)
        "roofline": dict(roofline_entry(
            "msa_decode_step: index_score_kernel + decode_fused_kernel<8,1,true> + "
            "decode_merge_kernel", layer_bytes, fused_ms, recorded_traffic("decode_step")),
            launches_per_step=3),
        "layer_step": {"algorithmic_bytes": layer_bytes,
                       "hbm_frac": frac(fused_ms),
                       "scoring_pass": roofline_entry("index_score_kernel", acc.score_bytes(cfg),
                                                      score_ms, recorded_traffic("index_score")),
                       "select_attend_merge_us": round((fused_ms - score_ms) * 1e3, 2),
                       # each layer-step timed on its own (an event pair per call)
                       "per_step_us": per_step,
                       "us_hip_graph": round(graph_ms * 1e3, 2),
                       "us_four_calls": round(four_ms * 1e3, 2),
                       "hbm_frac_four_calls": frac(four_ms),
                       "decode_attention_call": roofline_entry(
                           "decode_page_kernel + decode_merge_kernel", acc.decode_attn_bytes(cfg),
                           attn_ms)},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, layers[0], args.cpu_seconds)
    # the step before the path: this batch's tokens into the caches (random
    # rows; measured after everything that reads these caches)
    append_lines = {cfg.name: append_line(cfg, layers, args.steps, fused)}
    del fused, four, layers
    torch.cuda.empty_cache()
    # the step's streams as three plain dependent reads: index keys, the
    # attended K/V (and q/out), the page partials the merge reads back
    chain = (acc.score_bytes(cfg), acc.decode_attn_bytes(cfg),
             cfg.total_q * cfg.num_q_heads * cfg.topk * (2 * cfg.head_dim + 4))
    ceil = measured_ceilings(chain)
    result["measured_ceilings"] = ceil
    result["layer_step"]["three_read_launches_over_step"] = round(
        ceil["three_read_launches_us"] / (result["ms_per_step"] * 1e3), 4)
    result["roofline"]["frac_of_measured"] = round(
        result["roofline"]["achieved"] / ceil["hbm_read_gbs"], 4)
    result["roofline"]["frac_of_measured_64mib"] = round(
        result["roofline"]["achieved"] / ceil["hbm_read_64mib_gbs"], 4)
    sp = result["layer_step"]["scoring_pass"]
    sp["frac_of_measured_64mib"] = round(sp["achieved"] / ceil["hbm_read_64mib_gbs"], 4)
    result["layer_step"]["hbm_frac_of_measured"] = round(
        result["layer_step"]["hbm_frac"] * acc.HBM_PEAK_GBS / ceil["hbm_read_gbs"], 4)

    if not args.no_also:
        also = {}

        cpu_cfg = {}  # the oracle's stages per workload (CPU baseline)
        want_cpu = not args.no_cpu_baseline

        def decode_line(c, n_layers, n_steps, graph=False, cpu=False, record=None):
            ls = make_layers(c, n_layers)
            if cpu and want_cpu:
                cpu_cfg[c.name] = cpu_stages(c, ls[0])
            f = [MsaStep(x, fused=True) for x in ls]
            fo = [MsaStep(x) for x in ls]
            ms_ = time_calls([st.run for st in f], n_steps, 4)
            ms4_ = time_calls([st.run for st in fo], n_steps, 4)
            b_ = acc.score_bytes(c) + acc.decode_attn_bytes(c)
            line = {"us_per_layer_step": round(ms_ * 1e3, 2),
                    "layer_step_hbm_frac": round(b_ / (ms_ * 1e-3) / 1e9 / acc.HBM_PEAK_GBS, 4),
                    "algorithmic_bytes": int(b_),
                    "us_four_calls": round(ms4_ * 1e3, 2), "layers": n_layers}
            if graph:  # launch-bound: the same steps replayed as one HIP graph per pass
                line["us_hip_graph"] = round(time_graph(f, 4 * n_layers, 2 * n_layers) * 1e3, 2)
            if record:  # HBM bytes per layer-step counted by rocprofv3 (null if stale)
                line["traffic"] = recorded_traffic(record)
            del f, fo, ls
            torch.cuda.empty_cache()
            return line

        # decode at 4096 tokens, batch 1 (2.6 MB: launch-bound)
        c1 = gen.config(1)
        also[c1.name] = decode_line(c1, 128, max(128, args.steps), graph=True, cpu=True)
        # the 60k decode with one index key per KV group (H_idx = H_kv): 558 MB
        cg = gen.config(2).with_idx_heads(gen.config(2).num_kv_heads)
        also["paged_decode_b8_ctx60k_per_group_index_keys"] = decode_line(cg, 4, max(40, args.steps // 4))
        # ragged decode: 16 sequences, 4096 .. 524,288 tokens, 128 flattened rows
        c5 = gen.config(5)
        also[c5.name] = decode_line(c5, 2, max(20, args.steps // 4), cpu=True,
                                    record="decode_step_ragged")
        # multi-query decode: 4 and 8 draft tokens per sequence on the 60k
        # workload, as msa_multi_query_step and as its three calls
        # (msa_index_score -> msa_topk_blocks -> msa_sparse_attn_prefill)
        import dataclasses
        for nd in (4, 8):
            cm = dataclasses.replace(gen.config(2), name=f"multi_query_decode_b8_ctx60k_{nd}drafts",
                                     n_new=[nd] * 8)
            lm = make_layers(cm, 4)
            sm = [MsaStep(x, multi=True) for x in lm]
            s3 = [MsaStep(x) for x in lm]
            n_m = max(20, args.steps // 4)
            msm = time_calls([st.run for st in sm], n_m, 4)
            ms3 = time_calls([st.run for st in s3], n_m, 4)
            # bytes: index keys once for all drafts, each (sequence, group)'s
            # union of selected blocks once (from each layer's own selection),
            # rows and partials per selection; averaged over the layers
            bm = sum(acc.score_bytes(cm) + acc.multi_query_attn_bytes(cm, st.sel.cpu().numpy())
                     for st in sm) / len(sm)
            also[cm.name] = {"us_per_layer_step": round(msm * 1e3, 2),
                             "us_per_query_token": round(msm * 1e3 / cm.total_q, 2),
                             "us_three_calls": round(ms3 * 1e3, 2),
                             "algorithmic_bytes": int(bm),
                             "layer_step_hbm_frac": round(bm / (msm * 1e-3) / 1e9 / acc.HBM_PEAK_GBS, 4),
                             "entry_point": "msa_multi_query_step", "layers": 4}
            del sm, s3, lm
            torch.cuda.empty_cache()
        # 1M-context decode, batch 4 (18 GB of K/V per layer): 2 layers
        c4 = gen.config(4)
        l4 = make_layers(c4, 2)
        if want_cpu:
            cpu_cfg[c4.name] = cpu_stages(c4, l4[0])
        f4 = [MsaStep(x, fused=True) for x in l4]
        s4 = [MsaStep(x) for x in l4]
        n4 = max(10, args.steps // 8)
        ms4 = time_calls([s.run for s in f4], n4, 2)
        score4 = time_calls([s.score for s in s4], n4, 2)
        b4 = acc.score_bytes(c4) + acc.decode_attn_bytes(c4)
        dense[c4.name] = dense_line(c4, l4, 6, ms4)
        also[c4.name] = {"us_per_layer_step": round(ms4 * 1e3, 2),
                         "layer_step_hbm_frac": round(b4 / (ms4 * 1e-3) / 1e9 / acc.HBM_PEAK_GBS, 4),
                         "algorithmic_bytes": int(b4),
                         "traffic": recorded_traffic("decode_step_1m"),
                         "us_four_calls": round(time_calls([s.run for s in s4], n4, 2) * 1e3, 2),
                         "scoring_pass": roofline_entry("index_score_kernel", acc.score_bytes(c4), score4)}
        del f4, s4, l4
        torch.cuda.empty_cache()
        # chunked prefill: 8192 new tokens on a 57,344-token prefix, 2 layers
        c3 = gen.config(3)
        l3 = make_layers(c3, 2)
        if want_cpu:
            cpu_cfg[c3.name] = cpu_stages(c3, l3[0], sample_queries=32)
        s3 = [MsaStep(x) for x in l3]
        n3 = max(8, args.steps // 25)
        # enough untimed steps (about 15 ms) for the clocks to settle after the
        # lighter decode workloads
        w3 = max(8, args.warmup // 2)
        ms3 = time_calls([s.run for s in s3], n3, w3)
        score3 = time_calls([s.score for s in s3], n3, w3)
        attn3 = time_calls([s.attend for s in s3], n3, w3)
        fl_attn, fl_score = acc.attn_flops(c3), acc.score_flops(c3)
        tf = lambda fl, ms_: fl / (ms_ * 1e-3) / 1e12
        also[c3.name] = {
            "tokens_per_s": round(c3.total_q / (ms3 * 1e-3), 1),
            "ms_per_step": round(ms3, 4),
            "sparse_attn_call_ms": round(attn3, 4),
            "sparse_attn_call_mfma_frac": round(tf(fl_attn, attn3) / acc.BF16_PEAK_TFLOPS, 4),
            "sparse_attn_call_mfma_frac_of_measured": round(tf(fl_attn, attn3) / ceil["mfma_bf16_tflops"], 4),
            # the call's own traffic: K/V once, query rows gathered per
            # (query, head, slot), partials written and read back, outputs
            "sparse_attn_call_traffic": {
                "algorithmic_bytes": acc.prefill_attn_bytes(c3),
                "achieved_gbs": round(acc.prefill_attn_bytes(c3) / (attn3 * 1e-3) / 1e9, 1),
                "frac_of_copy_ceiling": round(acc.prefill_attn_bytes(c3) / (attn3 * 1e-3) / 1e9
                                              / ceil["hbm_copy_800mib_gbs"], 4)},
            "index_score_ms": round(score3, 4),
            "index_score_mfma_frac": round(tf(fl_score, score3) / acc.BF16_PEAK_TFLOPS, 4),
            "index_score_mfma_frac_of_measured": round(tf(fl_score, score3) / ceil["mfma_bf16_tflops"], 4),
            "index_score_rate_vs_vendor_gemm_randn": round(
                tf(fl_score, score3) / ceil["vendor_gemm_bf16_randn_tflops"], 4),
            "attn_flops": fl_attn, "score_flops": fl_score}
        # dense causal prefill baseline on the same chunk
        dfn = []
        for x in l3:
            d3 = _lib.dims_for(c3)
            o3 = torch.empty_like(x.q)
            e3 = torch.empty(x.q.shape[:2], dtype=torch.float32, device="cuda")
            dfn.append(lambda x=x, d3=d3, o3=o3, e3=e3: _lib.msa_dense_attn_prefill(
                d3, c3.total_q, x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, x.cu_q,
                o3, e3))
        dms3 = time_calls(dfn, max(4, n3 // 2), 1)
        fl_dense = acc.dense_prefill_flops(c3)
        also["dense_causal_prefill"] = {c3.name: {
            "ms": round(dms3, 4), "flops": fl_dense,
            "mfma_frac": round(tf(fl_dense, dms3) / acc.BF16_PEAK_TFLOPS, 4),
            "mfma_frac_of_measured": round(tf(fl_dense, dms3) / ceil["mfma_bf16_tflops"], 4),
            "rate_vs_vendor_gemm_randn": round(tf(fl_dense, dms3) / ceil["vendor_gemm_bf16_randn_tflops"], 4),
            "msa_step_speedup": round(dms3 / ms3, 2),
            "msa_sparse_attn_call_speedup": round(dms3 / attn3, 2)}}
        del dfn
        topk_line[c3.name] = topk_vs_torch(s3, n3)
        also["topk_vs_torch"] = topk_line
        append_lines[c3.name] = append_line(c3, l3, n3)
        also["cache_append"] = append_lines
        also["dense_gqa_decode"] = dense
        del s3, l3
        torch.cuda.empty_cache()
        result["also"] = also
        if want_cpu:
            cb = result["cpu_baseline"]
            cb["per_config"] = {cfg.name: cb.pop("stages"), **cpu_cfg}

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
