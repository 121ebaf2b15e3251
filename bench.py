"""Benchmark of the CSA decode hot path on one MI355X.

A step is one pass of the whole hot path over one batch: compression of the
blocks the step completes (none at the decode positions used here), the
Lightning Indexer, top-k and attention over the selected entries plus the
window.  The default workload is CSA decode at a 131072-token context:
batch 32, bf16 compressed KV (32768 entries, d=128), indexer 64 x 128,
top-k 1024, 64 query heads, window 128.  Inputs are seeded synthetic data
already resident in HBM when the timed region starts.

Prints one JSON line.  Only one GPU is supported.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="csa_decode_128k_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="launch stages directly, no HIP graphs")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="budget for the CPU oracle sample")
    return ap.parse_args()


def indexer_bytes(cfg, V: int) -> int:
    """Algorithmic HBM bytes of one indexer launch: every visible key once,
    one fp32 score written per entry, the queries and head weights."""
    key_bytes = cfg.d_I * (1 if cfg.ki_fp8 else 2 if cfg.storage == "bf16" else 4)
    per_entry = key_bytes + 4 + (4 if cfg.ki_fp8 else 0)
    q_bytes = cfg.T * cfg.H_I * (cfg.d_I * (1 if cfg.ki_fp8 else 2) + 4 + (4 if cfg.ki_fp8 else 0))
    return cfg.B * (V * per_entry + q_bytes)


def hca_bytes(cfg, V: int) -> int:
    """Algorithmic HBM bytes of one HCA attention launch: every visible K/V
    entry and window row once, queries in, fp32 outputs out."""
    eb = 2 if cfg.storage == "bf16" else 4
    return cfg.B * ((V + cfg.W) * 2 * cfg.d * eb + cfg.T * cfg.H * cfg.d * (eb + 4))


def cpu_baseline(cfg, budget_s: float):
    """The fp64 oracle on the host cores over a bounded sample of sequences."""
    import numpy as np
    import oracle
    import workloads as WL
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    done, t_total = 0, 0.0
    for b in range(cfg.B):
        s = WL.make_sequence(cfg, b)
        t0 = time.perf_counter()
        dec = oracle.bf16_decode if s["kc"].dtype == np.uint16 else (lambda a: a.astype(np.float64))
        pos = cfg.pos0 + np.arange(cfg.T)
        kc, vc = dec(s["kc"]), dec(s["vc"])
        if cfg.hca:
            oracle.hca_attend(dec(s["q"]), kc, vc, dec(s["kr"]), dec(s["vr"]), cfg.raw_pos0, pos,
                              cfg.m, cfg.W, cfg.scale)
        else:
            qi, ki = dec(s["qi"]), kc
            if cfg.ki_fp8:
                kcode, ksc = oracle.quantize_fp8_rows(kc.astype(np.float32))
                qcode, qsc = oracle.quantize_fp8_rows(qi.astype(np.float32))
                ki = oracle.e4m3_decode(kcode) * ksc[:, None]
                qi = oracle.e4m3_decode(qcode) * qsc[..., None]
            S = oracle.indexer_scores(qi, s["w"], ki, pos, cfg.m)
            V = oracle.visible_count(pos, cfg.m)
            idx = np.stack([oracle.topk_select(S[i], int(V[i]), cfg.k) for i in range(cfg.T)])
            oracle.attend(dec(s["q"]), kc, vc, idx, dec(s["kr"]), dec(s["vr"]), cfg.raw_pos0, pos,
                          cfg.W, cfg.scale)
        t_total += time.perf_counter() - t0
        done += 1
        if t_total >= budget_s:
            break
    q = done * cfg.T
    return {"value": q / t_total, "unit": "queries/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {cfg.B} sequences ({q} queries) of {cfg.name}, fp64 NumPy, "
                      f"{t_total:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the hot path has no multi-GPU mode)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import workloads as WL
    if not os.path.exists(os.path.join(ROOT, "long_context_sparse_16_amd", "libcsa.so")):
        import __graft_entry__
        __graft_entry__._build_module().build()
    from long_context_sparse_16_amd.pipeline import CSAStep

    cfg = WL.BY_NAME[args.workload]
    batch = WL.make_batch(cfg)
    step = CSAStep(cfg, batch)
    del batch
    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()

    # one HIP graph per stage: replays carry almost no host launch cost, and
    # events between replays on the same stream time each stage
    stages = ([step.compress] if cfg.n_new_tokens else []) + \
        ([step.index, step.topk] if not cfg.hca else []) + [step.attend]
    names = (["compress"] if cfg.n_new_tokens else []) + \
        (["index", "topk"] if not cfg.hca else []) + ["attend"]
    run_stage = stages
    if not args.eager:
        graphs = []
        for fn in stages:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn()
            graphs.append(g)
        run_stage = [g.replay for g in graphs]
        for _ in range(args.warmup):
            for r in run_stage:
                r()
        torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    K = args.steps
    n_ev = len(run_stage) + 1
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        e = ev[s]
        e[0].record(stream)
        for j, r in enumerate(run_stage):
            r()
            e[j + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    def stage(a, b):
        return float(np.mean([ev[s][a].elapsed_time(ev[s][b]) for s in range(K)]))

    st = {nm: stage(j, j + 1) for j, nm in enumerate(names)}
    st["step_events"] = stage(0, n_ev - 1)
    queries = cfg.B * cfg.T
    V = int(min(cfg.n_cap, (cfg.pos0 + cfg.T) // cfg.m))
    ms_per_step = wall * 1e3 / K
    value = queries * K / wall
    if cfg.hca:
        kb = hca_bytes(cfg, V)
        roof = {"kernel": "attend_kernel (HCA)", "bound": "hbm", "achieved": kb / (st["attend"] * 1e6),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "traffic": None}
    else:
        ib = indexer_bytes(cfg, V)
        roof = {"kernel": "indexer_kernel", "bound": "hbm", "achieved": ib / (st["index"] * 1e6),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "traffic": None}
    roof["frac"] = roof["achieved"] / roof["peak"]
    line = {
        "metric": "CSA decode queries/s (+ indexer entries scored/s) at 128K ctx",
        "value": value,
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if cfg.ki_fp8 else cfg.storage,
        "data": "synthetic (seeded N(0,1) K/V/q, U(0,1) head weights, planted entries)",
        "config": {"workload": cfg.name, "batch": cfg.B, "context_tokens": cfg.pos0,
                   "compressed_entries": V, "m": cfg.m, "indexer": f"{cfg.H_I}x{cfg.d_I}",
                   "top_k": cfg.k, "heads": cfg.H, "head_dim": cfg.d, "window": cfg.W},
        "entries_scored_per_s": (cfg.B * cfg.T * V * K / wall) if not cfg.hca else None,
        "stage_ms": st,
        "launch": "eager" if args.eager else "hip_graph_per_stage",
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
