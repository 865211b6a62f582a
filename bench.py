#!/usr/bin/env python3
"""Benchmark one MSA layer-step on one MI355X and print ONE JSON line.

Headline workload: paged decode, 8 sequences at a 60,000-token cached prefix,
H_q = 48, H_kv = 8, head_dim 128, idx_dim 64, Bk = 128, k = 16, physical pages
randomly permuted, keys given a per-block scale (seeded synthetic bf16 data).
A step is the whole hot path: msa_index_score -> msa_topk_blocks ->
msa_build_page_table -> msa_sparse_attn_decode, inputs resident in HBM.

Timing.  Every timed step starts from a cold cache: a 1 GiB read pass runs
before it (untimed), so the step's inputs come from HBM and not from the
256 MB Infinity Cache.  Each step is bracketed by HIP events on the stream
the kernels run on; ``value`` is the mean over the K timed steps of the step
replayed as one HIP graph.  The same steps launched eagerly, and warm-cache
back-to-back rates, are reported alongside.  The roofline kernel's duration
comes from events around its own call in the eager cold pass.

Also reported (``also``): 1M-context decode (batch 4), with its scoring pass
measured separately, and 8192-token chunked prefill onto a 57,344-token
prefix (tokens/s).  The oracle's CPU time on the headline workload is
reported as ``cpu_baseline``.
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
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-also", action="store_true", help="headline workload only")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="rough CPU budget for the oracle baseline")
    return ap.parse_args()


class Timer:
    """Cold-cache, per-step HIP-event timing of an MsaStep (eager and graph)."""

    def __init__(self, step, flush_bytes=1 << 30):
        import torch
        self.torch = torch
        self.step = step
        self.flush_buf = torch.ones(flush_bytes // 4, dtype=torch.float32, device="cuda")
        self.order = ["score", "topk"] + (["page_table"] if step.decode else []) + ["attend"]
        self.calls = {"score": step.score, "topk": step.topk, "attend": step.attend,
                      "page_table": getattr(step, "page_table_step", None)}
        self.graph = None

    def _ev(self):
        return self.torch.cuda.Event(enable_timing=True)

    def flush(self):
        # a read-only pass over 1 GiB evicts the step's inputs from the caches
        # without leaving dirty lines whose write-back would slow the step
        self.flush_sink = self.flush_buf.sum()

    def eager_cold(self, steps, probe):
        """Mean step ms and mean probe-call ms, each step after a cache flush."""
        torch = self.torch
        rec = []
        torch.cuda.synchronize()
        for _ in range(steps):
            self.flush()
            a, b, pa, pb = self._ev(), self._ev(), self._ev(), self._ev()
            a.record()
            for name in self.order:
                if name == probe:
                    pa.record()
                    self.calls[name]()
                    pb.record()
                else:
                    self.calls[name]()
            b.record()
            rec.append((a, b, pa, pb))
        torch.cuda.synchronize()
        step_ms = sum(a.elapsed_time(b) for a, b, _, _ in rec) / steps
        probe_ms = sum(pa.elapsed_time(pb) for _, _, pa, pb in rec) / steps
        return step_ms, probe_ms

    def per_call_cold(self, reps):
        torch = self.torch
        out = {}
        for name in self.order:
            evs = []
            for _ in range(reps):
                self.flush()
                a, b = self._ev(), self._ev()
                # the calls before `name` run first so its inputs are current
                for n2 in self.order:
                    if n2 == name:
                        a.record()
                        self.calls[n2]()
                        b.record()
                        break
                    self.calls[n2]()
                evs.append((a, b))
            torch.cuda.synchronize()
            out[name] = sum(a.elapsed_time(b) for a, b in evs) / reps
        return out

    def capture(self):
        torch = self.torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            self.step.run()  # warm the capture stream
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step.run()
        torch.cuda.synchronize()
        self.graph = g
        return g

    def graph_cold(self, steps):
        torch = self.torch
        g = self.graph or self.capture()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        rec = []
        for _ in range(steps):
            self.flush()
            a, b = self._ev(), self._ev()
            a.record()
            g.replay()
            b.record()
            rec.append((a, b))
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in rec) / steps

    def graph_warm(self, steps):
        torch = self.torch
        g = self.graph or self.capture()
        torch.cuda.synchronize()
        a, b = self._ev(), self._ev()
        a.record()
        for _ in range(steps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    def eager_warm(self, steps):
        torch = self.torch
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            self.step.run()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps


def cpu_baseline(cfg, x, budget_s):
    """The oracle (as it stands) on the same decode workload, full layer-steps."""
    import oracle
    from block_sparse_attention_03_amd import inputs as gen
    host = {k: gen.bits(getattr(x, k)) for k in
            ("q_idx", "kidx_cache", "q", "k_cache", "v_cache", "block_table", "seq_lens", "cu_q")}
    oracle.build(force=False)
    H = cfg.num_kv_heads

    def one_step():
        seq_of, pos_of = oracle.positions(host["seq_lens"], host["cu_q"])
        sc = oracle.index_score(host["q_idx"], host["kidx_cache"], host["block_table"], seq_of,
                                pos_of, cfg.block_size)
        sel = oracle.topk(sc, oracle.b_loc_rows(pos_of, H, cfg.block_size), cfg.topk)
        sel = sel.reshape(cfg.total_q, H, cfg.topk)
        oracle.page_table(sel, host["block_table"], host["seq_lens"], cfg.block_size)
        oracle.attention(host["q"], host["k_cache"], host["v_cache"], host["block_table"],
                         seq_of, pos_of, sel)

    n, t0 = 0, time.perf_counter()
    while True:
        one_step()
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 200:
            break
    return {"value": round(el * 1e6 / n, 1), "unit": "us/layer-step", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": f"{n} full layer-steps of the headline workload (64 rows scored over "
                      f"60,000 tokens each, top-k, page table, attention), fp64 C with OpenMP, "
                      f"{el:.1f} s"}


def roofline_entry(name, nbytes, ms, traffic=None):
    from block_sparse_attention_03_amd.accounting import HBM_PEAK_GBS
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "kernel": name, "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
            "algorithmic_bytes": int(nbytes), "avg_ms": round(ms, 5)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build has no "
              f"multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    from block_sparse_attention_03_amd import _lib, accounting as acc
    from block_sparse_attention_03_amd import inputs as gen
    from block_sparse_attention_03_amd.pipeline import MsaStep
    _lib.lib()  # fail loudly if the HIP library is missing

    # ---------------- headline: paged decode at 60k, batch 8 ----------------
    cfg = gen.config(2)
    x = gen.make_inputs(cfg, device="cuda")
    step = MsaStep(x)
    tm = Timer(step)
    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()
    calls = tm.per_call_cold(10)
    kernels = {"score": ("index_score_kernel", acc.score_bytes(cfg)),
               "attend": ("decode_page_kernel + decode_merge_kernel", acc.decode_attn_bytes(cfg))}
    probe = max(kernels, key=lambda k: calls[k])
    eager_ms, probe_ms = tm.eager_cold(args.steps, probe)
    graph_ms = tm.graph_cold(args.steps)
    layer_bytes = acc.score_bytes(cfg) + acc.decode_attn_bytes(cfg)

    def frac(ms_):
        return round(layer_bytes / (ms_ * 1e-3) / 1e9 / acc.HBM_PEAK_GBS, 4)

    result = {
        "metric": METRIC,
        "value": round(graph_ms * 1e3, 2),
        "unit": "us/layer-step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(graph_ms, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "num_seqs": cfg.num_seqs, "context": cfg.seq_lens[0],
                   "num_q_heads": cfg.num_q_heads, "num_kv_heads": cfg.num_kv_heads,
                   "num_idx_heads": cfg.num_idx_heads, "head_dim": cfg.head_dim,
                   "idx_dim": cfg.idx_dim, "block_size": cfg.block_size, "topk": cfg.topk,
                   "seed": cfg.seed, "cache": "cold (1 GiB read pass before each step)",
                   "launch": "HIP graph replay of the 4 ABI calls"},
        "roofline": roofline_entry(kernels[probe][0], kernels[probe][1], probe_ms),
        "layer_step": {"algorithmic_bytes": layer_bytes,
                       "hbm_frac_graph_cold": frac(graph_ms),
                       "us_eager_cold": round(eager_ms * 1e3, 2), "hbm_frac_eager_cold": frac(eager_ms),
                       "us_graph_warm": round(tm.graph_warm(args.steps) * 1e3, 2),
                       "us_eager_warm": round(tm.eager_warm(args.steps) * 1e3, 2),
                       "per_call_us_cold": {k: round(v * 1e3, 2) for k, v in calls.items()}},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, x, args.cpu_seconds)
    del tm, step, x
    torch.cuda.empty_cache()

    if not args.no_also:
        also = {}
        # 1M-context decode, batch 4: scoring pass reported on its own
        c4 = gen.config(4)
        x4 = gen.make_inputs(c4, device="cuda")
        s4 = MsaStep(x4)
        t4 = Timer(s4)
        s4.run()
        n4 = max(10, args.steps // 4)
        eager4, score4 = t4.eager_cold(n4, "score")
        graph4 = t4.graph_cold(n4)
        b4 = acc.score_bytes(c4) + acc.decode_attn_bytes(c4)
        also[c4.name] = {"us_per_layer_step": round(graph4 * 1e3, 2),
                         "layer_step_hbm_frac": round(b4 / (graph4 * 1e-3) / 1e9 / acc.HBM_PEAK_GBS, 4),
                         "us_eager_cold": round(eager4 * 1e3, 2),
                         "scoring_pass": roofline_entry("index_score_kernel", acc.score_bytes(c4), score4),
                         "per_call_us_cold": {k: round(v * 1e3, 2) for k, v in t4.per_call_cold(3).items()}}
        del t4, s4, x4
        torch.cuda.empty_cache()
        # chunked prefill: 8192 new tokens on a 57,344-token prefix
        c3 = gen.config(3)
        x3 = gen.make_inputs(c3, device="cuda")
        s3 = MsaStep(x3)
        t3 = Timer(s3)
        s3.run()
        n3 = max(5, args.steps // 20)
        eager3, attn3 = t3.eager_cold(n3, "attend")
        graph3 = t3.graph_cold(n3)
        calls3 = t3.per_call_cold(3)
        fl_attn, fl_score = acc.attn_flops(c3), acc.score_flops(c3)
        tf = lambda fl, ms_: fl / (ms_ * 1e-3) / 1e12
        also[c3.name] = {
            "tokens_per_s": round(c3.total_q / (graph3 * 1e-3), 1),
            "ms_per_step": round(graph3, 4), "ms_eager_cold": round(eager3, 4),
            "sparse_attn_call_mfma_frac": round(tf(fl_attn, attn3) / acc.BF16_PEAK_TFLOPS, 4),
            "index_score_mfma_frac": round(tf(fl_score, calls3["score"]) / acc.BF16_PEAK_TFLOPS, 4),
            "attn_flops": fl_attn, "score_flops": fl_score,
            "per_call_us_cold": {k: round(v * 1e3, 2) for k, v in calls3.items()}}
        del t3, s3, x3
        torch.cuda.empty_cache()
        result["also"] = also

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
