"""Benchmark of the CSA decode hot path on one MI355X.

A step is one pass of the whole hot path over one batch: compression of the
blocks the step completes (none at the decode positions used here), the
Lightning Indexer, top-k and attention over the selected entries plus the
window.  The default workload is CSA decode at a 131072-token context:
batch 32, bf16 compressed KV (32768 entries, d=128), indexer 64 x 128,
top-k 1024, 64 query heads, window 128.  The 1M-token decode workloads (CSA
with fp8 indexer keys, batch 4; HCA at m' = 128, batch 16) are timed in the
same run and reported under "workloads".  Inputs are seeded synthetic data
already resident in HBM when the timed region starts.

Timing is cold-cache: before every timed step (and every per-stage sample) a
1 GiB buffer is copied into another (1 GiB read + 1 GiB written, outside the
events), which evicts the 256 MB Infinity Cache and the L2s; each step is
bracketed by its own pair of HIP events on the launch stream, and the median
(p10, p90) is reported.  Back-to-back warm steps are reported as context.

Prints one JSON line.  Only one GPU is supported.
"""

from __future__ import annotations

import argparse
import glob
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "mxfp4": 10100.0, "f32": 157.3}
FLUSH_BYTES = 1 << 30
DEFAULT_WORKLOAD = "csa_decode_128k_bf16"
# timed in the same run as the default workload: the 1M-token half of the
# metric, and the chunked prefill (the indexer's MFMA fraction)
EXTRA_WORKLOADS = ("csa_decode_1m_fp8", "hca_decode_1m_bf16", "csa_chunked_prefill_256k_8k_bf16")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-extra", action="store_true",
                    help="time only --workload (not the 1M-token decode and chunked-prefill workloads)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="budget for the CPU oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (for HBM counter scaling)")
    return ap.parse_args()


# ------------------------------------------------------------ HBM counters

CSRC = os.path.join(ROOT, "long_context_sparse_16_amd", "csrc")
TRAFFIC_GLOB = os.path.join(ROOT, "profiles", "*_traffic.md")


def source_digest(paths) -> str:
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def kernel_sources(kernel: str) -> list:
    """The source files a kernel's machine code depends on."""
    main = {"indexer_kernel": "indexer.hip", "indexer_prefill_kernel": "indexer.hip",
            "attend_kernel": "attend.hip", "attend_merge_kernel": "attend.hip",
            "topk_classify_kernel": "topk.hip", "topk_finish_kernel": "topk.hip",
            "topk_row_kernel": "topk.hip"}[kernel]
    return [os.path.join(CSRC, f) for f in (main, "common.h", "kernels.h")]


def traffic_summaries() -> list:
    """The key/value block of every committed counter summary."""
    out = []
    for path in sorted(glob.glob(TRAFFIC_GLOB)):
        t = {"file": os.path.basename(path)}
        with open(path) as f:
            for line in f:
                if line.startswith("- ") and ": " in line:
                    key, val = line[2:].strip().split(": ", 1)
                    t[key] = val
        out.append(t)
    return out


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` in `workload` from the committed
    rocprofv3 counter summary (FETCH_SIZE + WRITE_SIZE per dispatch, each
    scaled by the same counter's reading for a plain copy of known size), or
    None when there is none or the kernel's sources changed since."""
    for t in traffic_summaries():
        if t.get("workload") != workload or t.get("kernel") != kernel:
            continue
        if t.get("source_sha256") != source_digest(kernel_sources(kernel)):
            return None
        return float(t["traffic_bytes_per_launch"])
    return None


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


# ------------------------------------------------------- algorithmic work

def visible(cfg, t: int) -> int:
    return max(0, min(cfg.n_cap, (t + 1) // cfg.m))


def visible_sum(cfg) -> int:
    """Sum over the step's queries of the causally visible entries V(t)."""
    return sum(visible(cfg, cfg.pos0 + i) for i in range(cfg.T))


def ki_row_bytes(cfg) -> int:
    """Bytes of one indexer key row with its scales."""
    if cfg.ki_mxfp4:
        return cfg.d_I // 2 + cfg.d_I // 32          # E2M1 codes + E8M0 scales
    if cfg.ki_fp8:
        return cfg.d_I + 4                           # E4M3 codes + fp32 scale
    return cfg.d_I * (2 if cfg.storage == "bf16" else 4)


def indexer_bytes(cfg) -> int:
    """Algorithmic HBM bytes of one indexer launch: every visible key (and
    its scales) read once per sequence, one fp32 score written per (query,
    visible entry), the queries (with their scales) and head weights read
    once."""
    V = visible(cfg, cfg.pos0 + cfg.T - 1)
    q_bytes = cfg.T * cfg.H_I * (ki_row_bytes(cfg) + 4)
    return cfg.B * (V * ki_row_bytes(cfg) + 4 * visible_sum(cfg) + q_bytes)


def step_bytes(cfg) -> int:
    """Algorithmic HBM bytes of one decode step: the indexer's key scan
    (with scales), the K/V rows each query attends (its top-k entries, or
    every visible entry for HCA, plus its window rows), the queries, head
    weights and the fp32 outputs.  The indexer's score round trip is not
    counted (it is the implementation's, not the method's)."""
    eb = 2 if cfg.storage == "bf16" else 4
    tot = 0
    for i in range(cfg.T):
        t = cfg.pos0 + i
        V = visible(cfg, t)
        keys = (V if cfg.hca else min(cfg.k, V)) + min(cfg.W, t + 1)
        q = cfg.H * cfg.d * eb + cfg.H * cfg.d * 4
        if cfg.k > 0:
            q += V * ki_row_bytes(cfg) + cfg.H_I * (ki_row_bytes(cfg) + 4)
        tot += keys * 2 * cfg.d * eb + q
    return cfg.B * tot


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
        tot += min(cfg.k, visible(cfg, t)) + min(cfg.W, t + 1)
    return 10 * cfg.d * cfg.H * cfg.B * tot


def hca_bytes(cfg) -> int:
    """Algorithmic HBM bytes of one HCA attention launch: every visible K/V
    entry and window row once, queries in, fp32 outputs out."""
    return step_bytes(cfg)


def hca_splits(cfg) -> int:
    """More than one when the HCA attention splits its rows over workgroups
    (a merge launch follows): the library then needs a partials workspace."""
    import long_context_sparse_16_amd as csa
    return 2 if csa.hca_attend_workspace_size(cfg.B, cfg.T, cfg.H, cfg.d, cfg.n_cap, cfg.W) > 0 else 1


# ------------------------------------------------------------ CPU baseline

def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(cfg, budget_s: float):
    """The fp64 oracle on the host cores over a bounded sample of sequences."""
    import numpy as np
    import workloads as WL
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    done, t_total = 0, 0.0
    layer_cfgs = WL.layer_workloads(cfg) if cfg.layers else [cfg]
    base = {"unit": "queries/s", "cores": int(threads), "cpu_model": cpu_model(), "kind": "oracle"}
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
        return {"value": n / dt, **base,
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
    return {"value": q / t_total, **base,
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


# ------------------------------------------------------------------ timing

class Timer:
    """Cold-cache event timing on one stream.  flush() (outside the events)
    overwrites a 1 GiB buffer with a copy of another and then reads the
    source back: afterwards no input of the timed work is left in the 256 MB
    Infinity Cache or the L2s, and the dirty lines the overwrite left in the
    Infinity Cache have been written back.  (Without the read-back, that
    write-back -- up to 256 MB -- lands inside the next timed kernel: a
    268 MB streaming read measured 49 us after copy + read, 78 us after the
    copy alone, 104 us after a 1 GiB fill, 43 us warm.)"""

    def __init__(self, torch, stream):
        self.torch = torch
        self.stream = stream
        self.src = torch.empty(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda:0").fill_(1)
        self.dst = torch.empty_like(self.src)
        self.sink = torch.empty((), dtype=torch.int64, device="cuda:0")

    def flush(self):
        self.dst.copy_(self.src)
        self.torch.sum(self.src, dim=(0,), dtype=self.torch.int64, out=self.sink)

    def samples(self, fn, n, cold=True, pre=None, post=None):
        """Durations (us) of n calls of fn, each between its own events;
        pre() / post() run outside the events."""
        torch = self.torch
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        for a, b in evs:
            if cold:
                self.flush()
            if pre:
                pre()
            a.record(self.stream)
            fn()
            b.record(self.stream)
            if post:
                post()
        torch.cuda.synchronize()
        return [a.elapsed_time(b) * 1e3 for a, b in evs]

    def staged(self, stages, n, cold=True):
        """Per-stage durations (us) of n cold passes over `stages` (a list of
        (name, fn)), with one event between consecutive stages."""
        torch = self.torch
        runs = []
        for _ in range(n):
            if cold:
                self.flush()
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
            evs[0].record(self.stream)
            for i, (_, fn) in enumerate(stages):
                fn()
                evs[i + 1].record(self.stream)
            runs.append(evs)
        torch.cuda.synchronize()
        return {name: [evs[i].elapsed_time(evs[i + 1]) * 1e3 for evs in runs]
                for i, (name, _) in enumerate(stages)}


    def kernel_samples(self, stages, target, n_kernels, n):
        """Kernel durations (us) of n cold passes over `stages`: from the
        start of the first to the end of the n_kernels-th kernel that stage
        `target` launches, recorded by those kernels' own launches
        (csa_time_next_kernels: hipExtLaunchKernelGGL start / stop events on
        the kernels' stream), so without the dispatch around the call."""
        import long_context_sparse_16_amd as csa
        torch = self.torch
        out = []
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(self.stream)  # creates the HIP events the launches record into
        b.record(self.stream)
        try:
            for _ in range(n):
                self.flush()
                for name, fn in stages:
                    if name == target:
                        csa.csa_time_next_kernels(a, b, n_kernels)
                    fn()
                torch.cuda.synchronize()
                out.append(a.elapsed_time(b) * 1e3)
        finally:
            csa.csa_time_next_kernels(None, None, 0)
        return out


def stats(xs) -> dict:
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90)), "mean": float(a.mean())}


def attainable_bandwidth(torch, timer) -> dict:
    """HBM bandwidth a plain device copy of 1 GiB reaches (read + write bytes,
    GB/s, median of 10 cold runs): a practical ceiling beside the nominal
    8 TB/s."""
    n = FLUSH_BYTES
    a = torch.empty(n // 4, dtype=torch.int32, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    cp = stats(timer.samples(lambda: b.copy_(a), 10))["median"]
    del a, b
    return {"copy_gbs": 2 * n / (cp * 1e3)}


# -------------------------------------------------------------- workloads

def make_step(cfg):
    """The step object, the function that runs one step, and the stages of a
    step as (name, fn) for per-stage timing."""
    import numpy as np
    import torch
    import workloads as WL
    from long_context_sparse_16_amd.pipeline import CSAStep, HybridStep
    if cfg.layers:
        layer_cfgs = WL.layer_workloads(cfg)
        h = HybridStep(layer_cfgs, [WL.make_batch(c) for c in layer_cfgs])
        stages = [(f"layer{i}_{k}", lay.run) for i, (k, lay) in enumerate(zip(cfg.layers, h.layers))]
        return h, h.run, stages
    batch = WL.make_batch(cfg)
    step = CSAStep(cfg, batch)
    del batch
    if cfg.backward:
        # the forward once (its outputs, lse and indices feed the backward),
        # then a seeded upstream gradient N(0, 1)
        step.run()
        g_rng = np.random.Generator(np.random.PCG64(cfg.seed))
        step.dout = torch.from_numpy(g_rng.standard_normal((cfg.B, cfg.T, cfg.H, cfg.d),
                                                           dtype=np.float32)).to("cuda:0")
        fn = lambda: step.backward(step.dout)  # noqa: E731
        return step, fn, [("backward", fn)]
    return step, step.run, step.stages()


def measure(cfg, K, W, timer, torch):
    """Cold and warm step times, per-stage times and the roofline of one
    workload."""
    obj, run, stages = make_step(cfg)
    for _ in range(W):
        timer.flush()
        run()
    torch.cuda.synchronize()
    cold = timer.samples(run, K)
    warm = timer.samples(run, max(10, K // 2), cold=False)
    st = timer.staged(stages, max(10, K // 2))
    st_stats = {k: stats(v) for k, v in st.items()}
    res = {"step_us": {**stats(cold), "warm_median": stats(warm)["median"]},
           "stage_us": {k: round(v["median"], 2) for k, v in st_stats.items()}}
    med = res["step_us"]["median"]
    res["queries_per_s"] = cfg.B * cfg.T / (med * 1e-6)
    n_indexed = (sum(1 for k in cfg.layers if k == "csa") if cfg.layers else 1) if cfg.k > 0 else 0
    if n_indexed and not cfg.backward:
        res["entries_scored_per_s"] = n_indexed * cfg.B * visible_sum(cfg) / (med * 1e-6)
    # roofline of the dominant kernel: the mean of its cold launches, timed
    # by the launches' own start / stop events (the kernel time a rocprofv3
    # kernel trace of this run averages); `call_frac` is the same bytes over
    # the event pair around the whole call (dispatch included)
    def kernel_mean(stage, n_kernels=1):
        return stats(timer.kernel_samples(stages, stage, n_kernels, max(10, K // 2)))["mean"]

    call_us = None
    if cfg.backward:
        fl = backward_flops(cfg)
        t_us = st_stats["backward"]["mean"]
        # bf16 storage: the products run on the bf16 MFMA (fp32 operands as
        # bf16 hi + lo pairs); fp32 storage: on the fp32 MFMA
        pk = "bf16" if cfg.storage == "bf16" else "f32"
        roof = {"kernel": "attend_bwd (rows + reductions)", "bound": "mfma",
                "achieved": fl / (t_us * 1e6), "peak": MFMA_PEAK_TFLOPS[pk],
                "unit": "TFLOP/s", "traffic": None, "algorithmic_flops": fl}
    elif cfg.layers:
        i = next(i for i, k in enumerate(cfg.layers) if k == "csa")
        lay = WL_layer(cfg, i)
        roof = {"kernel": f"layer {i} (csa) step", "bound": "hbm", "unit": "GB/s",
                "achieved": step_bytes(lay) / (st_stats[f"layer{i}_csa"]["mean"] * 1e3),
                "peak": HBM_PEAK_GBS, "traffic": None, "algorithmic_bytes": step_bytes(lay)}
    elif cfg.hca:
        kb = hca_bytes(cfg)
        # the attention launch and, when the rows are split, the merge
        n_k = 2 if hca_splits(cfg) > 1 else 1
        t_us, call_us = kernel_mean("attend", n_k), st_stats["attend"]["mean"]
        roof = {"kernel": "attend_kernel (HCA) + merge" if n_k == 2 else "attend_kernel (HCA)",
                "bound": "hbm", "achieved": kb / (t_us * 1e3), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "traffic": measured_traffic(cfg.name, "attend_kernel"),
                "algorithmic_bytes": kb}
    elif cfg.T >= 8:
        fl = indexer_flops(cfg)
        t_us, call_us = kernel_mean("index"), st_stats["index"]["mean"]
        roof = {"kernel": "indexer_prefill_kernel", "bound": "mfma",
                "achieved": fl / (t_us * 1e6),
                "peak": MFMA_PEAK_TFLOPS[index_dtype(cfg)], "unit": "TFLOP/s",
                "traffic": None, "algorithmic_flops": fl}
    else:
        ib = indexer_bytes(cfg)
        stage = "index" if "index" in st_stats else "select"
        t_us, call_us = kernel_mean(stage), st_stats[stage]["mean"]
        roof = {"kernel": "indexer_kernel", "bound": "hbm",
                "achieved": ib / (t_us * 1e3), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "traffic": measured_traffic(cfg.name, "indexer_kernel"),
                "algorithmic_bytes": ib}
    roof["frac"] = roof["achieved"] / roof["peak"]
    if call_us is not None:
        roof["kernel_us"] = t_us
        roof["call_us"] = call_us
        roof["call_frac"] = roof["frac"] * t_us / call_us
    if cfg.T == 1 and not cfg.backward:
        sb = step_bytes(cfg) if not cfg.layers else sum(
            step_bytes(WL_layer(cfg, i)) for i in range(len(cfg.layers)))
        roof["step_bytes"] = sb
        roof["step_gbs"] = sb / (med * 1e3)
        roof["step_frac"] = roof["step_gbs"] / HBM_PEAK_GBS
    res["roofline"] = roof
    del obj, run, stages
    return res


def WL_layer(cfg, i):
    import workloads as WL
    return WL.layer_workloads(cfg)[i]


def config_of(cfg) -> dict:
    V = visible(cfg, cfg.pos0 + cfg.T - 1)
    return {"workload": cfg.name, "batch": cfg.B, "query_tokens": cfg.T,
            "context_tokens": cfg.pos0, "compressed_entries": V, "m": cfg.m,
            "indexer": f"{cfg.H_I}x{cfg.d_I}" if cfg.k else None,
            "indexer_dtype": index_dtype(cfg) if cfg.k else None,
            "top_k": cfg.k, "heads": cfg.H, "head_dim": cfg.d, "window": cfg.W,
            **({"layers": list(cfg.layers)} if cfg.layers else {})}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the hot path has no multi-GPU mode)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    import torch

    import workloads as WL
    import __graft_entry__
    __graft_entry__._build_module().ensure_current()
    cfg = WL.BY_NAME[args.workload]
    stream = torch.cuda.current_stream()
    timer = Timer(torch, stream)
    attain = attainable_bandwidth(torch, timer)

    K = args.steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    main_res = measure(cfg, K, args.warmup, timer, torch)
    wall = time.perf_counter() - t0
    torch.cuda.empty_cache()
    extra = {}
    if not args.no_extra and cfg.name == DEFAULT_WORKLOAD:
        for name in EXTRA_WORKLOADS:
            ec = WL.BY_NAME[name]
            r = measure(ec, K, args.warmup, timer, torch)
            extra[name] = {"config": config_of(ec), **r}
            torch.cuda.empty_cache()

    med_ms = main_res["step_us"]["median"] * 1e-3
    roof = main_res.pop("roofline")
    roof["attainable"] = attain
    line = {
        "metric": "CSA decode queries/s + indexer entries scored/s at 128K/1M ctx; % HBM/MFMA peak",
        "value": main_res.pop("queries_per_s"),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": med_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if cfg.backward else index_dtype(cfg),
        "data": "synthetic (seeded N(0,1) K/V/q, U(0,1) head weights, planted entries)",
        "config": config_of(cfg),
        "timing": "cold cache: a 1 GiB device copy and a read-back of its source before every timed step, outside the events; "
                  "one event pair per step on the launch stream; value = queries / median step",
        **main_res,
        "timed_region_s": wall,
        "roofline": roof,
        "workloads": extra,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
