"""Seeded synthetic inputs for the CSA / HCA hot path.

This module is shared by the tests, the benchmark and the smoke check.  It
holds no part of the method's arithmetic: it only draws random numbers,
rounds them to the storage format (through PyTorch's own bf16 conversion)
and places "planted" high-affinity keys.  Both the HIP library and the CPU
oracle consume exactly the bytes produced here.

Workload shapes follow the pages' V4-Pro parameters (m = 4, indexer 64 heads
x 128, top-k 1024, window 128, HCA m' = 128; "DeepSeek V4 technical review",
takeshell.com, sections 2.1 and 2.2) at 128K and 1M-token contexts.  The
pages' long-context quality suites are not used; these synthetic contexts
stand in for them by shape only.

Recipe (per workload, seed = 1600 + workload number, one child
``SeedSequence`` per batch sequence so any sequence can be regenerated
alone): values ~ N(0, 1) (head weights ~ U(0, 1)) drawn in float32 in a fixed
order, then rounded to nearest-even bf16 where the workload stores bf16.
Planted keys: with u = sum_h w_h * q_I[h] (the weighted indexer query, from
the stored values) and g the key row already drawn at that index,
key = |g| * (0.9 * u/|u| + sqrt(0.19) * g_perp/|g_perp|), g_perp being the
part of g orthogonal to u; the result is then rounded to bf16.
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    number: int                # seed = 1600 + number
    B: int                     # sequences in the batch
    T: int                     # query tokens per sequence
    pos0: int                  # absolute position of the first query token
    m: int                     # compression ratio (m' for HCA)
    d: int                     # head dim of the shared KV head and of q
    H: int                     # query heads
    W: int                     # sliding window length
    n_ctx_entries: int         # compressed entries that already exist
    n_new_tokens: int          # raw tokens compressed inside the step
    raw_before: int            # raw context tokens kept before the first query
    H_I: int = 0               # indexer heads (0: HCA, no indexer)
    d_I: int = 0
    k: int = 0                 # top-k (0: HCA)
    storage: str = "bf16"      # "f32" or "bf16" (K/V, q, q_I)
    ki_fp8: bool = False       # indexer keys / queries stored as e4m3 + scale
    ki_mxfp4: bool = False     # indexer keys / queries stored as MXFP4
    swa: bool = False          # sliding-window-only attention (no compressed entries read)
    layers: tuple = ()         # hybrid stack: per-layer kinds "swa" / "csa" / "hca"
    block_end: bool = False    # decode token completes a block: the step compresses
                               # it into entry n_ctx_entries (logits for every raw row)
    backward: bool = False     # the timed step is the backward pass of the forward step
    planted: int = 0           # planted high-affinity entries per sequence
    planted_spread: bool = False  # evenly spaced (else seeded distinct random)
    description: str = ""

    @property
    def seed(self) -> int:
        return 1600 + self.number

    @property
    def hca(self) -> bool:
        return self.k == 0 and not self.swa

    @property
    def n_cap(self) -> int:
        return self.n_ctx_entries + self.n_new_tokens // self.m + (1 if self.block_end else 0)

    @property
    def raw_pos0(self) -> int:
        return self.pos0 - self.raw_before

    @property
    def R(self) -> int:
        return self.raw_before + self.T

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads, then the MXFP4 variant of the 1M decode.  Decode
# queries sit at position t = context length
# (the new token is the last raw token of the window); the chunked prefill's
# queries are the 8192 appended tokens.
TINY_PREFILL_F32 = Workload(
    name="csa_prefill_2k_f32", number=0, B=1, T=2048, pos0=0, m=4, d=64, H=8,
    W=32, n_ctx_entries=0, n_new_tokens=2048, raw_before=0, H_I=4, d_I=64,
    k=64, storage="f32",
    description="tiny CSA prefill, fp32: n=2048, m=4, d=64, indexer 4x64, "
                "top-k 64, 8 query heads, window 32")
DECODE_128K_BF16 = Workload(
    name="csa_decode_128k_bf16", number=1, B=32, T=1, pos0=131072, m=4,
    d=128, H=64, W=128, n_ctx_entries=32768, n_new_tokens=0, raw_before=127,
    H_I=64, d_I=128, k=1024, storage="bf16", planted=16,
    description="CSA decode, bf16 KV: batch 32 x 131072 tokens (32768 "
                "entries), indexer 64x128, top-k 1024, 64 heads x 128, "
                "window 128, 16 planted entries per sequence")
PREFILL_256K_BF16 = Workload(
    name="csa_chunked_prefill_256k_8k_bf16", number=2, B=1, T=8192,
    pos0=262144, m=4, d=128, H=64, W=128, n_ctx_entries=65536,
    n_new_tokens=8192, raw_before=127, H_I=64, d_I=128, k=1024,
    storage="bf16",
    description="CSA chunked prefill, bf16: 8192 new tokens on a 262144-token "
                "context (65536 + 2048 entries), indexer 64x128, top-k 1024")
HCA_DECODE_1M_BF16 = Workload(
    name="hca_decode_1m_bf16", number=3, B=16, T=1, pos0=1048576, m=128,
    d=128, H=64, W=128, n_ctx_entries=8192, n_new_tokens=0, raw_before=127,
    storage="bf16",
    description="HCA decode, bf16: batch 16 x 1048576 tokens at m'=128 (8192 "
                "entries), dense over all entries + window 128, 64 heads")
DECODE_1M_FP8 = Workload(
    name="csa_decode_1m_fp8", number=4, B=4, T=1, pos0=1048576, m=4, d=128,
    H=64, W=128, n_ctx_entries=262144, n_new_tokens=0, raw_before=127,
    H_I=64, d_I=128, k=1024, storage="bf16", ki_fp8=True, planted=64,
    planted_spread=True,
    description="CSA decode at 1M, fp8 e4m3 indexer keys/queries with fp32 "
                "row scales: batch 4 x 262144 entries, top-k 1024, 64 planted")

DECODE_1M_MXFP4 = DECODE_1M_FP8.replace(
    name="csa_decode_1m_mxfp4", number=5, ki_fp8=False, ki_mxfp4=True,
    description="CSA decode at 1M, MXFP4 indexer keys/queries (E2M1 + E8M0 "
                "per 32): batch 4 x 262144 entries, top-k 1024, 64 planted")

# A hybrid stack of attention layers for one decode token ("DeepSeek V4
# technical review", takeshell.com, 2.3 "Hybrid Architecture Design": the
# first 2 layers are pure sliding-window attention, then CSA and HCA
# alternate).  Every layer has its own caches; the layer count (8) is this
# build's choice (the pages give none).
HYBRID_DECODE_128K_BF16 = DECODE_128K_BF16.replace(
    name="hybrid_decode_128k_bf16", number=6,
    layers=("swa", "swa", "csa", "hca", "csa", "hca", "csa", "hca"),
    description="hybrid decode stack, bf16: 2 sliding-window layers then CSA / HCA "
                "alternating (8 layers, own caches each), batch 32 x 131072 tokens")

# The 128K decode at a step whose token completes a block: t = 131071, so
# (t + 1) % 4 == 0 and block 32767 (positions 131068 .. 131071, the last 4
# raw rows) is compressed inside the step and is visible to its own query.
DECODE_128K_BF16_BLOCK_END = DECODE_128K_BF16.replace(
    name="csa_decode_128k_bf16_block_end", number=7, pos0=131071, n_ctx_entries=32767,
    block_end=True,
    description="CSA decode, bf16, at a block boundary: the step compresses the block "
                "its token completes (entry 32767) and scores it with the 32767 older "
                "entries; otherwise as csa_decode_128k_bf16")

# The backward pass of the chunked prefill's attention and compression (the
# training-shaped step: 8192 query tokens over 67584 entries, top-1024 +
# window 128, 64 heads x 128), with a seeded upstream gradient N(0, 1).
PREFILL_256K_BF16_BACKWARD = PREFILL_256K_BF16.replace(
    name="csa_chunked_prefill_256k_8k_bf16_backward", number=8, backward=True,
    description="backward pass of the chunked prefill (csa_chunked_prefill_256k_8k_bf16): "
                "attention gradients for 8192 query tokens and the compressor gradients of "
                "the chunk's 2048 new entries")

WORKLOADS = [TINY_PREFILL_F32, DECODE_128K_BF16, PREFILL_256K_BF16,
             HCA_DECODE_1M_BF16, DECODE_1M_FP8, DECODE_1M_MXFP4, HYBRID_DECODE_128K_BF16,
             DECODE_128K_BF16_BLOCK_END, PREFILL_256K_BF16_BACKWARD]
BY_NAME = {w.name: w for w in WORKLOADS}


def bf16_codes(x) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest-even, PyTorch's conversion)
    and return the uint16 codes."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_values(codes) -> np.ndarray:
    """float32 values of bf16 codes (the top half of a float32 word)."""
    c = np.ascontiguousarray(codes, dtype=np.uint16)
    return (c.astype(np.uint32) << 16).view(np.float32)


def _normal(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32)


def _store(cfg: Workload, x):
    """Storage form of a float32 draw: float32 itself or bf16 codes."""
    return x.astype(np.float32) if cfg.storage == "f32" else bf16_codes(x)


def _values(cfg: Workload, stored):
    return stored if cfg.storage == "f32" else bf16_values(stored)


def _planted_rows(cfg: Workload, rng, n_entries: int) -> np.ndarray:
    if cfg.planted == 0:
        return np.zeros(0, dtype=np.int64)
    if cfg.planted_spread:
        i = np.arange(cfg.planted)
        return ((i + 0.5) * n_entries / cfg.planted).astype(np.int64)
    return np.sort(rng.choice(n_entries, size=cfg.planted, replace=False)).astype(np.int64)


def _plant(key_rows: np.ndarray, u: np.ndarray) -> np.ndarray:
    """Rotate each row g toward u: |g| (0.9 u_hat + sqrt(0.19) g_perp_hat)."""
    u = u.astype(np.float64)
    uh = u / np.linalg.norm(u)
    g = key_rows.astype(np.float64)
    gn = np.linalg.norm(g, axis=1, keepdims=True)
    gp = g - (g @ uh)[:, None] * uh[None, :]
    gp /= np.linalg.norm(gp, axis=1, keepdims=True)
    return (gn * (0.9 * uh[None, :] + np.sqrt(0.19) * gp)).astype(np.float32)


def make_sequence(cfg: Workload, b: int) -> dict:
    """All inputs of sequence ``b`` of ``cfg`` as NumPy arrays in storage form
    (float32, or uint16 bf16 codes).  Keys:

    kc, vc     [n_ctx_entries, d]   pre-existing compressed cache (may be empty)
    kr, vr     [R, d]               raw K/V at positions raw_pos0 .. pos0+T-1
    z          [n_new_tokens, d]    compressor logits (float32) for the raw
                                    tokens pos0 .. pos0+n_new_tokens-1
                                    (block_end: [R, d], one row per raw row)
    qi         [T, H_I, d_I]        indexer queries (absent for HCA)
    w          [T, H_I]             indexer head weights, float32
    q          [T, H, d]            attention queries
    planted    [P]                  indices of planted entries
    """
    ss = np.random.SeedSequence(cfg.seed).spawn(cfg.B)[b]
    rng = np.random.Generator(np.random.PCG64(ss))
    out = {}
    d = cfg.d
    kc = _normal(rng, (cfg.n_ctx_entries, d))
    vc = _normal(rng, (cfg.n_ctx_entries, d))
    kr = _normal(rng, (cfg.R, d))
    vr = _normal(rng, (cfg.R, d))
    z = _normal(rng, (cfg.R if cfg.block_end else cfg.n_new_tokens, d))
    q = _normal(rng, (cfg.T, cfg.H, d))
    if cfg.k > 0:
        qi = _normal(rng, (cfg.T, cfg.H_I, cfg.d_I))
        w = rng.random((cfg.T, cfg.H_I), dtype=np.float32)
        out["qi"] = _store(cfg, qi)
        out["w"] = w
    planted = _planted_rows(cfg, rng, cfg.n_ctx_entries)
    if planted.size:
        # u from the stored (rounded) indexer query of the first query token
        qv = _values(cfg, out["qi"])[0].astype(np.float64)
        u = (out["w"][0].astype(np.float64)[:, None] * qv).sum(axis=0)
        kc[planted] = _plant(kc[planted], u)
    out["kc"] = _store(cfg, kc)
    out["vc"] = _store(cfg, vc)
    out["kr"] = _store(cfg, kr)
    out["vr"] = _store(cfg, vr)
    out["z"] = z
    out["q"] = _store(cfg, q)
    out["planted"] = planted
    return out


def make_batch(cfg: Workload, sequences=None) -> dict:
    """Stack ``make_sequence`` over the batch (or the listed sequences)."""
    seqs = range(cfg.B) if sequences is None else sequences
    per = [make_sequence(cfg, b) for b in seqs]
    return {key: np.stack([p[key] for p in per]) for key in per[0]}


def layer_workloads(cfg: Workload) -> list:
    """The per-layer workloads of a hybrid stack: each has its own seed
    (number 100 * cfg.number + layer).  CSA layers keep cfg's indexer and
    top-k; HCA layers compress at m' = 128 (entries = context / 128);
    sliding-window layers read only the window (one placeholder entry)."""
    out = []
    for i, kind in enumerate(cfg.layers):
        base = cfg.replace(name=f"{cfg.name}/{i}:{kind}", number=100 * cfg.number + i, layers=())
        if kind == "csa":
            out.append(base)
        elif kind == "hca":
            out.append(base.replace(m=128, n_ctx_entries=cfg.pos0 // 128, H_I=0, d_I=0, k=0,
                                    planted=0))
        elif kind == "swa":
            out.append(base.replace(n_ctx_entries=1, H_I=0, d_I=0, k=0, planted=0, swa=True))
        else:
            raise ValueError(kind)
    return out


def tiny(cfg: Workload, **kw) -> Workload:
    """A reduced copy of a workload for parity tests at oracle-friendly sizes."""
    return cfg.replace(**kw)
