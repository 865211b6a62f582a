#!/usr/bin/env python3
"""Benchmark one MSA layer-step on one MI355X and print ONE JSON line.

Headline workload: paged decode, 8 sequences at a 60,000-token cached prefix,
H_q = 48, H_kv = 8, head_dim 128, idx_dim 64, Bk = 128, k = 16, physical pages
randomly permuted, keys given a per-block scale (seeded synthetic bf16 data).
A step is the whole hot path: msa_index_score -> msa_topk_blocks ->
msa_build_page_table -> msa_sparse_attn_decode, inputs resident in HBM.

Also reported (``also``): 1M-context decode (batch 4), with its scoring pass
measured separately, and 8192-token chunked prefill onto a 57,344-token
prefix (tokens/s).  Kernel durations come from HIP events recorded on the
stream the kernels run on, inside the timed region.

The oracle's CPU time on the same workload is reported as ``cpu_baseline``.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "MSA decode µs/layer-step & prefill tok/s at 60k/1M ctx; % HBM/MFMA peak"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-also", action="store_true", help="headline workload only")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="rough CPU budget for the oracle baseline")
    return ap.parse_args()


def timed_steps(step, steps, warmup, probe):
    """Run warmup, then `steps` timed steps; events bracket the `probe` call."""
    import torch
    for _ in range(warmup):
        step.run()
    torch.cuda.synchronize()
    calls = {"score": step.score, "topk": step.topk, "attend": step.attend}
    if step.decode:
        calls["page_table"] = step.page_table_step
    order = ["score", "topk"] + (["page_table"] if step.decode else []) + ["attend"]
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        for name in order:
            if name == probe:
                ev[i][0].record()
                calls[name]()
                ev[i][1].record()
            else:
                calls[name]()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    probe_ms = sum(a.elapsed_time(b) for a, b in ev) / steps
    return (t1 - t0) * 1e3 / steps, probe_ms


def per_call_ms(step, reps=20):
    """Average duration of every ABI call of the step (events, outside the timed region)."""
    import torch
    names = ["score", "topk"] + (["page_table"] if step.decode else []) + ["attend"]
    fns = {"score": step.score, "topk": step.topk, "attend": step.attend,
           "page_table": getattr(step, "page_table_step", None)}
    out = {}
    for name in names:
        evs = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fns[name]()
            b.record()
            evs.append((a, b))
        torch.cuda.synchronize()
        out[name] = sum(a.elapsed_time(b) for a, b in evs) / reps
    return out


def cpu_baseline(cfg, x, budget_s):
    """The oracle (as it stands) on the same decode workload, full layer-steps."""
    import numpy as np

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
        if el >= budget_s or n >= 50:
            break
    return {"value": round(el * 1e6 / n, 1), "unit": "us/layer-step", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": f"{n} full layer-steps of the headline workload (all 64 rows scored over "
                      f"60,000 tokens, top-k, page table, attention), fp64 C + OpenMP, "
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
    step.run()
    torch.cuda.synchronize()
    calls = per_call_ms(step)
    by_bytes = {"score": acc.score_bytes(cfg), "attend": acc.decode_attn_bytes(cfg)}
    probe = max(("score", "attend"), key=lambda k: calls[k])
    ms, probe_ms = timed_steps(step, args.steps, args.warmup, probe)
    layer_bytes = acc.score_bytes(cfg) + acc.decode_attn_bytes(cfg)
    kernel_names = {"score": "index_score_kernel", "attend": "decode_page_kernel + decode_merge_kernel"}
    result = {
        "metric": METRIC,
        "value": round(ms * 1e3, 2),
        "unit": "us/layer-step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "num_seqs": cfg.num_seqs, "context": cfg.seq_lens[0],
                   "num_q_heads": cfg.num_q_heads, "num_kv_heads": cfg.num_kv_heads,
                   "num_idx_heads": cfg.num_idx_heads, "head_dim": cfg.head_dim,
                   "idx_dim": cfg.idx_dim, "block_size": cfg.block_size, "topk": cfg.topk,
                   "seed": cfg.seed},
        "roofline": roofline_entry(kernel_names[probe], by_bytes[probe], probe_ms),
        "layer_step": {"algorithmic_bytes": layer_bytes,
                       "hbm_frac": round(layer_bytes / (ms * 1e-3) / 1e9 / acc.HBM_PEAK_GBS, 4),
                       "per_call_ms": {k: round(v, 5) for k, v in calls.items()}},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, x, args.cpu_seconds)
    del step, x
    torch.cuda.empty_cache()

    if not args.no_also:
        also = {}
        # 1M-context decode, batch 4: scoring pass reported on its own
        c4 = gen.config(4)
        x4 = gen.make_inputs(c4, device="cuda")
        s4 = MsaStep(x4)
        ms4, score_ms = timed_steps(s4, max(10, args.steps // 4), 3, "score")
        calls4 = per_call_ms(s4, reps=5)
        b4 = acc.score_bytes(c4) + acc.decode_attn_bytes(c4)
        also[c4.name] = {"us_per_layer_step": round(ms4 * 1e3, 2),
                         "layer_step_hbm_frac": round(b4 / (ms4 * 1e-3) / 1e9 / acc.HBM_PEAK_GBS, 4),
                         "scoring_pass": roofline_entry("index_score_kernel", acc.score_bytes(c4), score_ms),
                         "per_call_ms": {k: round(v, 5) for k, v in calls4.items()}}
        del s4, x4
        torch.cuda.empty_cache()
        # chunked prefill: 8192 new tokens on a 57,344-token prefix
        c3 = gen.config(3)
        x3 = gen.make_inputs(c3, device="cuda")
        s3 = MsaStep(x3)
        ms3, attn_ms = timed_steps(s3, max(5, args.steps // 20), 2, "attend")
        calls3 = per_call_ms(s3, reps=5)
        fl_attn = acc.attn_flops(c3)
        fl_score = acc.score_flops(c3)
        also[c3.name] = {
            "tokens_per_s": round(c3.total_q / (ms3 * 1e-3), 1),
            "ms_per_step": round(ms3, 4),
            "sparse_attn_mfma_frac": round(fl_attn / (attn_ms * 1e-3) / 1e12 / acc.BF16_PEAK_TFLOPS, 4),
            "index_score_mfma_frac": round(fl_score / (calls3["score"] * 1e-3) / 1e12 / acc.BF16_PEAK_TFLOPS, 4),
            "attn_flops": fl_attn, "score_flops": fl_score,
            "per_call_ms": {k: round(v, 5) for k, v in calls3.items()}}
        del s3, x3
        torch.cuda.empty_cache()
        result["also"] = also

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
