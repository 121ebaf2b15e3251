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
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "mxfp4": 10100.0, "f32": 157.3}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="csa_decode_128k_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="replay one HIP graph per step instead of launching each stage "
                         "directly (slower here: each graph replay adds ~13 us)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="budget for the CPU oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (for HBM counter scaling)")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "indexer_decode_128k_traffic.md")
INDEXER_SOURCES = [os.path.join(ROOT, "long_context_sparse_16_amd", "csrc", f)
                   for f in ("indexer.hip", "common.h", "kernels.h")]


def source_digest(paths) -> str:
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(cfg):
    """HBM bytes per indexer launch from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE per dispatch, each scaled by the same
    counter's reading for a plain copy of known size), or None when the
    summary is for another workload or for a different indexer source."""
    t = {}
    try:
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if line.startswith("- ") and ": " in line:
                    key, val = line[2:].strip().split(": ", 1)
                    t[key] = val
    except OSError:
        return None
    if t.get("workload") != cfg.name or t.get("source_sha256") != source_digest(INDEXER_SOURCES):
        return None
    return float(t["traffic_bytes_per_launch"])


def copy_calibration():
    """A plain device copy of 256 MiB, five times (rocprofv3 counters of
    this copy scale FETCH_SIZE / WRITE_SIZE to bytes)."""
    import torch
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "copies": 5}), flush=True)


def visible_sum(cfg) -> int:
    """Sum over the step's queries of the causally visible entries V(t)."""
    return sum(min(cfg.n_cap, (cfg.pos0 + i + 1) // cfg.m) for i in range(cfg.T))


def indexer_bytes(cfg, V: int) -> int:
    """Algorithmic HBM bytes of one indexer launch: every visible key (and
    its fp8 scale or MXFP4 block scales) read once per sequence, one fp32
    score written per (query, visible entry), the queries (with their
    scales) and head weights read once."""
    if cfg.ki_mxfp4:
        row = cfg.d_I // 2 + cfg.d_I // 32          # E2M1 codes + E8M0 scales
    elif cfg.ki_fp8:
        row = cfg.d_I + 4                           # E4M3 codes + fp32 scale
    else:
        row = cfg.d_I * (2 if cfg.storage == "bf16" else 4)
    q_bytes = cfg.T * cfg.H_I * (row + 4)
    return cfg.B * (V * row + 4 * visible_sum(cfg) + q_bytes)


def index_dtype(cfg) -> str:
    return "mxfp4" if cfg.ki_mxfp4 else "fp8" if cfg.ki_fp8 else cfg.storage


def indexer_flops(cfg) -> int:
    """Algorithmic flops of one indexer launch: a d_I-long dot product per
    (query, indexer head, visible entry)."""
    return 2 * cfg.B * cfg.H_I * cfg.d_I * visible_sum(cfg)


def backward_flops(cfg) -> int:
    """Algorithmic FLOP of the attention backward: 10 d per (query row, key,
    head) -- the logits, dP, dq, dK and dV products -- over every query's
    key list (min(k, V(t)) selected entries plus its window rows)."""
    tot = 0
    for i in range(cfg.T):
        t = cfg.pos0 + i
        V = min(cfg.n_cap, (t + 1) // cfg.m)
        tot += min(cfg.k, V) + min(cfg.W, t + 1)
    return 10 * cfg.d * cfg.H * cfg.B * tot


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
    layer_cfgs = WL.layer_workloads(cfg) if cfg.layers else [cfg]
    if cfg.T >= 8:
        # prefill-shaped: a sample of query rows (i = 31 mod 32) of the first
        # sequence, grown while the budget lasts
        s = WL.make_sequence(cfg, 0)
        sample = np.arange(31, cfg.T, 32)
        n = 4
        while True:
            t0 = time.perf_counter()
            _oracle_sequence(cfg, s, rows=sample[:n])
            dt = time.perf_counter() - t0
            if dt * 2 > budget_s or n >= sample.size:
                break
            n = min(sample.size, n * 2)
        return {"value": n / dt, "unit": "queries/s", "cores": int(threads), "kind": "oracle",
                "sample": f"{n} query rows (i = 31 mod 32) of sequence 0 of {cfg.name}, fp64 "
                          f"NumPy, {dt:.1f} s"}
    # the batch's sequences in turn (again from the first once all are
    # done) until the budget is spent
    while True:
        b = done % cfg.B
        for lc in layer_cfgs:
            s = WL.make_sequence(lc, b)
            t0 = time.perf_counter()
            _oracle_sequence(lc, s)
            t_total += time.perf_counter() - t0
        done += 1
        if t_total >= budget_s:
            break
    q = done * cfg.T
    return {"value": q / t_total, "unit": "queries/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} sequence steps ({q} queries; the batch's {cfg.B} sequences in "
                      f"turn) of {cfg.name}, fp64 NumPy, {t_total:.1f} s"}


def _oracle_sequence(cfg, s, rows=None):
    """The oracle's whole step for one sequence's inputs ``s`` (query rows
    ``rows`` only, when given)."""
    import numpy as np
    import oracle
    dec = oracle.bf16_decode if s["kc"].dtype == np.uint16 else (lambda a: a.astype(np.float64))
    rows = np.arange(cfg.T) if rows is None else np.asarray(rows)
    pos = cfg.pos0 + rows
    kc, vc = dec(s["kc"]), dec(s["vc"])
    if cfg.n_new_tokens:
        # the step's own tokens, compressed and appended
        r0, r1 = cfg.raw_before, cfg.raw_before + cfg.n_new_tokens
        kc = np.vstack([kc, oracle.compress(dec(s["kr"][r0:r1]), s["z"], cfg.m)])
        vc = np.vstack([vc, oracle.compress(dec(s["vr"][r0:r1]), s["z"], cfg.m)])
    q = dec(s["q"])[rows]
    if cfg.block_end:
        # the block completed by the query token: its last m raw rows
        r0 = cfg.R - cfg.m
        z = s["z"][r0:]
        kc = np.vstack([kc, oracle.compress(dec(s["kr"][r0:]), z, cfg.m)])
        vc = np.vstack([vc, oracle.compress(dec(s["vr"][r0:]), z, cfg.m)])
    if cfg.hca:
        oracle.hca_attend(q, kc, vc, dec(s["kr"]), dec(s["vr"]), cfg.raw_pos0, pos,
                          cfg.m, cfg.W, cfg.scale)
    elif cfg.swa:
        idx = np.zeros((rows.size, 0), np.int64)
        oracle.attend(q, kc, vc, idx, dec(s["kr"]), dec(s["vr"]), cfg.raw_pos0, pos,
                      cfg.W, cfg.scale)
    else:
        qi, ki = dec(s["qi"])[rows], kc
        if cfg.ki_fp8:
            kcode, ksc = oracle.quantize_fp8_rows(kc.astype(np.float32))
            qcode, qsc = oracle.quantize_fp8_rows(qi.astype(np.float32))
            ki = oracle.e4m3_decode(kcode) * ksc[:, None]
            qi = oracle.e4m3_decode(qcode) * qsc[..., None]
        if cfg.ki_mxfp4:
            ki = oracle.mxfp4_decode_rows(*oracle.quantize_mxfp4_rows(kc.astype(np.float32)))
            qi = oracle.mxfp4_decode_rows(*oracle.quantize_mxfp4_rows(qi.astype(np.float32)))
        S = oracle.indexer_scores(qi, s["w"][rows], ki, pos, cfg.m)
        V = oracle.visible_count(pos, cfg.m)
        idx = np.stack([oracle.topk_select(S[i], int(V[i]), cfg.k) for i in range(rows.size)])
        oracle.attend(q, kc, vc, idx, dec(s["kr"]), dec(s["vr"]), cfg.raw_pos0, pos,
                      cfg.W, cfg.scale)
        if cfg.backward:
            g_rng = np.random.Generator(np.random.PCG64(cfg.seed))
            dout = g_rng.standard_normal((cfg.T, cfg.H, cfg.d), dtype=np.float32)[rows]
            g = oracle.attend_backward(q, kc, vc, idx, dec(s["kr"]), dec(s["vr"]), cfg.raw_pos0,
                                       pos, cfg.W, cfg.scale, dout)
            if cfg.n_new_tokens:
                r0, r1 = cfg.raw_before, cfg.raw_before + cfg.n_new_tokens
                for x, dc in ((s["kr"], g["dkc"]), (s["vr"], g["dvc"])):
                    oracle.compress_backward(dec(x[r0:r1]), s["z"], cfg.m,
                                             dc[cfg.n_ctx_entries:cfg.n_cap])


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the hot path has no multi-GPU mode)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    import numpy as np
    import torch

    import workloads as WL
    if not os.path.exists(os.path.join(ROOT, "long_context_sparse_16_amd", "libcsa.so")):
        import __graft_entry__
        __graft_entry__._build_module().build()
    from long_context_sparse_16_amd.pipeline import CSAStep

    cfg = WL.BY_NAME[args.workload]
    if cfg.layers:
        # hybrid stack: every layer runs in the step; the stage timings and
        # the roofline are those of its first CSA layer
        from long_context_sparse_16_amd.pipeline import HybridStep
        layer_cfgs = WL.layer_workloads(cfg)
        hstep = HybridStep(layer_cfgs, [WL.make_batch(c) for c in layer_cfgs])
        run_once = hstep.run
        first_csa = next(i for i, c in enumerate(layer_cfgs) if c.k > 0)
        step, rcfg = hstep.layers[first_csa], layer_cfgs[first_csa]
    else:
        batch = WL.make_batch(cfg)
        step = CSAStep(cfg, batch)
        del batch
        run_once, rcfg = step.run, cfg
        if cfg.backward:
            # the forward once (its outputs, lse and indices feed the
            # backward), then a seeded upstream gradient N(0, 1)
            step.run()
            g_rng = np.random.Generator(np.random.PCG64(cfg.seed))
            dout = torch.from_numpy(g_rng.standard_normal((cfg.B, cfg.T, cfg.H, cfg.d),
                                                          dtype=np.float32)).to("cuda:0")

            def run_once():
                step.backward(dout)
    for _ in range(args.warmup):
        run_once()
    torch.cuda.synchronize()

    # The timed step launches each stage directly on the current stream
    # (--graph: one HIP graph per step instead).  Each stage is also timed on
    # its own with events over back-to-back calls; the dominant kernel's
    # duration for the roofline comes from those.
    stream = torch.cuda.current_stream()
    if not args.graph:
        run_step = run_once
    else:
        g_step = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_step):
            run_once()
        run_step = g_step.replay
        for _ in range(args.warmup):
            run_step()
    torch.cuda.synchronize()

    K = args.steps
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(K):
        run_step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_event_ms = ev0.elapsed_time(ev1) / K

    # per-stage timing: R back-to-back calls of one stage (--graph: one graph
    # holding them).
    # The indexer also accumulates the top-k histogram into the top-k
    # workspace, which only the following top-k call consumes: the index
    # stage is timed alone and the workspace cleared afterwards, and top-k
    # is timed as (index + top-k) minus index.
    import long_context_sparse_16_amd as csa_lib

    def timed(fn, R=20, reps=3):
        """Per-call time of fn: one graph holding R calls back to back,
        replayed `reps` times between events (default: R*reps direct calls)."""
        if not args.graph:
            def rep():
                for _ in range(R):
                    fn()
        else:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(R):
                    fn()
            rep = g.replay
        rep()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            rep()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / (R * reps)

    st = {}
    if cfg.layers:
        for i, lay in enumerate(hstep.layers):
            st[f"layer{i}_{cfg.layers[i]}"] = timed(lay.run)
    cfg_all, cfg = cfg, rcfg  # stage timings and roofline: the (first CSA) layer
    if cfg.backward:
        csa_lib_ = __import__("long_context_sparse_16_amd")
        st["attend_backward"] = timed(lambda: csa_lib_.csa_attend_backward(
            step.q, step.kc, step.vc, step.idx, step.kr, step.vr, step.raw_pos0, step.pos0,
            cfg.W, cfg.scale, step.out, step.lse, dout, ws=step.bwd_ws), R=5, reps=2)
        st["backward_step"] = step_event_ms
    elif cfg.n_new_tokens:
        st["compress"] = timed(step.compress)
    if cfg.k > 0 and not cfg.backward:
        st["index"] = timed(step.index)
        csa_lib.csa_workspace_clear(step.topk_ws)

        def index_topk():
            step.index()
            step.topk()
        st["topk"] = timed(index_topk) - st["index"]
    if not cfg.backward:
        st["attend"] = timed(step.attend)
    if cfg.block_end:
        # the fused selection (block compression inside the indexer launch,
        # then top-k) against the same step with separate compress launches
        st["select_fused"] = timed(step.select)
        st["compress_unfused"] = timed(step.compress)
        st["step_unfused"] = timed(step.run_unfused)
    st["step_events"] = step_event_ms
    cfg = cfg_all

    queries = cfg.B * cfg.T
    n_indexed = ((sum(1 for k in cfg.layers if k == "csa") if cfg.layers else 1)
                 if cfg.k > 0 and not cfg.backward else 0)
    V = int(min(cfg.n_cap, (cfg.pos0 + cfg.T) // cfg.m))
    ms_per_step = wall * 1e3 / K
    value = queries * K / wall
    if cfg.backward:
        # the attention backward's products (S, dP, dq, dK, dV: 10 d FLOP per
        # query row, key and head) on the fp32 MFMA, against the whole call
        # (row kernel + the two deterministic reductions)
        fl = backward_flops(cfg)
        roof = {"kernel": "attend_bwd (rows + reductions)", "bound": "mfma",
                "achieved": fl / (st["attend_backward"] * 1e9), "peak": MFMA_PEAK_TFLOPS["f32"],
                "unit": "TFLOP/s", "traffic": None, "algorithmic_flops": fl}
    elif cfg.hca:
        kb = hca_bytes(cfg, V)
        roof = {"kernel": "attend_kernel (HCA)", "bound": "hbm", "achieved": kb / (st["attend"] * 1e6),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "traffic": None}
    elif cfg.T >= 8:
        # prefill: the indexer is one MFMA score GEMM per sequence
        fl = indexer_flops(cfg)
        dt = index_dtype(cfg)
        roof = {"kernel": "indexer_prefill_kernel", "bound": "mfma",
                "achieved": fl / (st["index"] * 1e9), "peak": MFMA_PEAK_TFLOPS[dt],
                "unit": "TFLOP/s", "traffic": None, "algorithmic_flops": fl}
    else:
        ib = indexer_bytes(cfg, V)
        roof = {"kernel": "indexer_kernel", "bound": "hbm", "achieved": ib / (st["index"] * 1e6),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "traffic": measured_traffic(cfg),
                "algorithmic_bytes": ib}
    roof["frac"] = roof["achieved"] / roof["peak"]
    line = {
        "metric": "CSA decode queries/s + indexer entries scored/s at 128K/1M ctx; % HBM/MFMA peak",
        "value": value,
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if cfg.backward else index_dtype(cfg),
        "data": "synthetic (seeded N(0,1) K/V/q, U(0,1) head weights, planted entries)",
        "config": {"workload": cfg.name, "batch": cfg.B, "context_tokens": cfg.pos0,
                   "compressed_entries": V, "m": cfg.m, "indexer": f"{cfg.H_I}x{cfg.d_I}",
                   "top_k": cfg.k, "heads": cfg.H, "head_dim": cfg.d, "window": cfg.W,
                   **({"layers": list(cfg.layers)} if cfg.layers else {})},
        "entries_scored_per_s": (n_indexed * cfg.B * visible_sum(cfg) * K / wall) if n_indexed else None,
        "stage_ms": st,
        "launch": "hip_graph_per_step" if args.graph else "direct",
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
