"""Parity of the backward pass (csa_attend_backward, hca_attend_backward,
csa_compress_backward) with the fp64 oracle's gradients, on inputs whose
forward the GPU computes (out, lse) and a seeded upstream gradient.  Sizes
span several key chunks, ragged index lists (-1 padding), windows cut at
position 0, heads below the kernel's 64 head slots, and the chunked-prefill
shape; two runs must give the same bits."""

import numpy as np
import pytest
import torch

from conftest import ensure_library
from gpu_util import DEV, bf16_codes, decode, from_dev, rel_l2, say, to_dev

import oracle
import workloads as WL

pytestmark = pytest.mark.gpu

ensure_library()
import long_context_sparse_16_amd as csa  # noqa: E402
from long_context_sparse_16_amd.pipeline import CSAStep  # noqa: E402


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _store(x, storage):
    return x.astype(np.float32) if storage == "f32" else bf16_codes(x)


# fp32 forward: outputs exact to ~1e-6, so the gradients are held to fp32
# accuracy; bf16 forward: its output carries the bf16 rounding of P in the
# PV product (2^-9 relative per probability), which enters D = dout . out
# and so ds, dq and dK (dV does not use it and stays at fp32 accuracy).
TOL = {"f32": (1e-5, 1e-5), "bf16": (5e-3, 1e-2)}   # (rel-L2, max-abs / max|ref|)


def _close(name, got, ref, storage):
    rl, ma = TOL[storage]
    r = rel_l2(got, ref)
    m = float(np.max(np.abs(got - ref))) / max(float(np.max(np.abs(ref))), 1e-30)
    say("  ", name, "rel-l2", r, "max-abs/max", m)
    assert r <= rl and m <= ma, (name, r, m)


def _case(rng, storage, B, T, H, d, n_cap, k, W, m, pos0s):
    R = T + W
    q = _store(rng.standard_normal((B, T, H, d)), storage)
    kc = _store(rng.standard_normal((B, n_cap, d)), storage)
    vc = _store(rng.standard_normal((B, n_cap, d)), storage)
    kr = _store(rng.standard_normal((B, R, d)), storage)
    vr = _store(rng.standard_normal((B, R, d)), storage)
    pos0 = np.asarray(pos0s, np.int64)
    raw_pos0 = pos0 + T - R                          # the raw rows end at the last query
    idx = np.full((B, T, k), -1, np.int32)
    for b in range(B):
        for i in range(T):
            V = int(min(n_cap, (pos0[b] + i + 1) // m))
            n = min(k, V) - (i % 3 == 1 and min(k, V) > 0)   # some rows ragged
            if n > 0:
                idx[b, i, :n] = np.sort(rng.choice(V, size=n, replace=False))
    dout = rng.standard_normal((B, T, H, d)).astype(np.float32)
    return q, kc, vc, kr, vr, pos0, raw_pos0, idx, dout


@pytest.mark.parametrize("storage,H,d", [("f32", 8, 64), ("f32", 64, 128), ("bf16", 64, 128),
                                         ("bf16", 20, 64)])
def test_csa_attend_backward_parity(storage, H, d):
    say("csa attend backward", storage, H, d)
    rng = np.random.default_rng(8000 + H + d)
    B, T, n_cap, k, W, m = 2, 37, 300, 40, 16, 4
    pos0s = [4, 4 * n_cap - T - 2]                    # windows cut at 0 / full cache
    q, kc, vc, kr, vr, pos0, raw_pos0, idx, dout = _case(rng, storage, B, T, H, d, n_cap, k, W, m,
                                                         pos0s)
    scale = 1.0 / np.sqrt(d)
    args = (to_dev(q), to_dev(kc), to_dev(vc), to_dev(idx), to_dev(kr), to_dev(vr),
            to_dev(raw_pos0), to_dev(pos0), W, scale)
    out, lse = csa.csa_attend(*args)
    g = csa.csa_attend_backward(*args, out, lse, to_dev(dout))
    g2 = csa.csa_attend_backward(*args, out, lse, to_dev(dout))
    torch.cuda.synchronize()
    for key in g:
        assert torch.equal(g[key], g2[key]), ("not reproducible", key)
    for b in range(B):
        pos = pos0[b] + np.arange(T)
        ref = oracle.attend_backward(decode(q[b]), decode(kc[b]), decode(vc[b]), idx[b],
                                     decode(kr[b]), decode(vr[b]), raw_pos0[b], pos, W, scale,
                                     dout[b])
        for key in ("dq", "dkc", "dvc", "dkr", "dvr"):
            _close(f"{key}[{b}]", from_dev(g[key])[b], ref[key], storage)


def test_csa_attend_backward_hot_entries():
    """Entries that every query row selects: 2304 references each, more
    than the small-list variant of the key/value reduction holds, so the
    large-list variant sorts and sums them."""
    say("csa attend backward, hot entries")
    rng = np.random.default_rng(8123)
    B, T, H, d, n_cap, k, W, m = 1, 2304, 8, 64, 600, 12, 8, 4
    pos0s = [4 * n_cap - 1]                          # every entry visible
    q, kc, vc, kr, vr, pos0, raw_pos0, idx, dout = _case(rng, "f32", B, T, H, d, n_cap, k, W, m,
                                                         pos0s)
    hot = np.array([0, 7, 300, 599], np.int32)
    for i in range(T):
        rest = rng.choice(np.setdiff1d(np.arange(n_cap), hot), size=k - hot.size, replace=False)
        idx[0, i] = np.sort(np.concatenate([hot, rest.astype(np.int32)]))
    scale = 1.0 / np.sqrt(d)
    args = (to_dev(q), to_dev(kc), to_dev(vc), to_dev(idx), to_dev(kr), to_dev(vr),
            to_dev(raw_pos0), to_dev(pos0), W, scale)
    out, lse = csa.csa_attend(*args)
    g = csa.csa_attend_backward(*args, out, lse, to_dev(dout))
    torch.cuda.synchronize()
    ref = oracle.attend_backward(q[0], kc[0], vc[0], idx[0], kr[0], vr[0], raw_pos0[0],
                                 pos0[0] + np.arange(T), W, scale, dout[0])
    for key in ("dkc", "dvc"):
        _close(f"{key} hot", from_dev(g[key])[0][hot], ref[key][hot], "f32")
        _close(key, from_dev(g[key])[0], ref[key], "f32")


@pytest.mark.parametrize("storage", ["f32", "bf16"])
def test_hca_attend_backward_parity(storage):
    say("hca attend backward", storage)
    rng = np.random.default_rng(8100)
    B, T, H, d, n_cap, W, m = 2, 21, 64, 128, 70, 8, 4
    pos0s = [0, 4 * n_cap - T - 1]
    q, kc, vc, kr, vr, pos0, raw_pos0, _, dout = _case(rng, storage, B, T, H, d, n_cap, 1, W, m,
                                                       pos0s)
    scale = 1.0 / np.sqrt(d)
    args = (to_dev(q), to_dev(kc), to_dev(vc), m, to_dev(kr), to_dev(vr), to_dev(raw_pos0),
            to_dev(pos0), W, scale)
    out, lse = csa.hca_attend(*args)
    g = csa.hca_attend_backward(*args, out, lse, to_dev(dout))
    torch.cuda.synchronize()
    for b in range(B):
        pos = pos0[b] + np.arange(T)
        ref = oracle.hca_attend_backward(decode(q[b]), decode(kc[b]), decode(vc[b]), decode(kr[b]),
                                         decode(vr[b]), raw_pos0[b], pos, m, W, scale, dout[b])
        for key in ("dq", "dkc", "dvc", "dkr", "dvr"):
            _close(f"{key}[{b}]", from_dev(g[key])[b], ref[key], storage)


@pytest.mark.parametrize("storage,m", [("f32", 4), ("bf16", 4), ("bf16", 128), ("f32", 1)])
def test_compress_backward_parity(storage, m):
    say("compress backward", storage, m)
    rng = np.random.default_rng(8200 + m)
    B, nb, d = 2, 9, 128
    x = _store(rng.standard_normal((B, nb * m, d)), storage)
    z = (rng.standard_normal((B, nb * m, d)) * 2).astype(np.float32)
    dc = rng.standard_normal((B, nb, d)).astype(np.float32)
    dx, dz = csa.csa_compress_backward(to_dev(x), to_dev(z), to_dev(dc), m)
    dx, dz = from_dev(dx), from_dev(dz)
    for b in range(B):
        rdx, rdz = oracle.compress_backward(decode(x[b]), z[b], m, dc[b])
        assert np.max(np.abs(dx[b] - rdx)) <= 1e-6 * max(1.0, np.max(np.abs(rdx)))
        assert np.max(np.abs(dz[b] - rdz)) <= 1e-5 * max(1.0, np.max(np.abs(rdz)))


def test_backward_tiny_prefill_f32_end_to_end():
    """The parity configuration (2048 tokens, fp32): forward through the
    pipeline, then the backward of its attention against the oracle's, and
    the compressor's backward fed the GPU's entry gradients."""
    cfg = WL.TINY_PREFILL_F32
    say("backward", cfg.name)
    batch = WL.make_batch(cfg)
    step = CSAStep(cfg, batch)
    step.run()
    rng = np.random.default_rng(8300)
    dout = rng.standard_normal(tuple(step.out.shape)).astype(np.float32)
    g = csa.csa_attend_backward(step.q, step.kc, step.vc, step.idx, step.kr, step.vr,
                                step.raw_pos0, step.pos0, cfg.W, cfg.scale, step.out, step.lse,
                                to_dev(dout))
    torch.cuda.synchronize()
    pos = cfg.pos0 + np.arange(cfg.T)
    kc, vc = from_dev(step.kc)[0].astype(np.float64), from_dev(step.vc)[0].astype(np.float64)
    ref = oracle.attend_backward(decode(batch["q"][0]), kc, vc, from_dev(step.idx)[0],
                                 decode(batch["kr"][0]), decode(batch["vr"][0]), cfg.raw_pos0, pos,
                                 cfg.W, cfg.scale, dout[0])
    for key in ("dq", "dkc", "dvc", "dkr", "dvr"):
        _close(key, from_dev(g[key])[0], ref[key], "f32")
    # the compressor's gradient for the entry gradients just computed
    dx, dz = csa.csa_compress_backward(step.kr, step.z, g["dkc"], cfg.m)
    rdx, rdz = oracle.compress_backward(decode(batch["kr"][0]), batch["z"][0], cfg.m,
                                        from_dev(g["dkc"])[0])
    assert np.max(np.abs(from_dev(dx)[0] - rdx)) <= 1e-5 * max(1.0, np.max(np.abs(rdx)))
    assert np.max(np.abs(from_dev(dz)[0] - rdz)) <= 1e-5 * max(1.0, np.max(np.abs(rdz)))


def test_backward_chunked_prefill_256k_sampled():
    """The backward of the chunked prefill at full size, in the launch
    configuration the benchmark times: dq on sampled query rows, the key /
    value gradients of sampled entries (old context, first and last new
    entry) and raw rows from the oracle over exactly the rows that attended
    them, and the compressor gradients of the chunk's new entries."""
    cfg = WL.PREFILL_256K_BF16_BACKWARD
    say("backward", cfg.name)
    batch = WL.make_batch(cfg)
    step = CSAStep(cfg, batch)
    step.run()
    g_rng = np.random.Generator(np.random.PCG64(cfg.seed))
    dout = g_rng.standard_normal((cfg.B, cfg.T, cfg.H, cfg.d), dtype=np.float32)
    g = step.backward(to_dev(dout))
    torch.cuda.synchronize()
    idx = from_dev(step.idx)[0]
    kc, vc = decode(from_dev(step.kc)[0]), decode(from_dev(step.vc)[0])
    q, kr, vr = decode(batch["q"][0]), decode(batch["kr"][0]), decode(batch["vr"][0])
    pos_all = cfg.pos0 + np.arange(cfg.T)

    def ref_over(rows):
        return oracle.attend_backward(q[rows], kc, vc, idx[rows], kr, vr, cfg.raw_pos0,
                                      pos_all[rows], cfg.W, cfg.scale, dout[0][rows])

    rows = np.array([0, 31, 4095, 8191])
    r = ref_over(rows)
    _close("dq rows", from_dev(g["dq"])[0][rows], r["dq"], "bf16")
    # old entries, the first and last new one, and the most attended new one
    new_users = [(idx == j).any(axis=1).sum() for j in range(cfg.n_ctx_entries, cfg.n_cap, 7)]
    j_hot = cfg.n_ctx_entries + 7 * int(np.argmax(new_users))
    for j in (0, 33333, cfg.n_ctx_entries, cfg.n_cap - 1, j_hot):
        users = np.nonzero((idx == j).any(axis=1))[0]
        say("  entry", j, "attended by", users.size, "rows")
        if users.size == 0:
            assert np.all(from_dev(g["dkc"])[0][j] == 0)
            continue
        r = ref_over(users)
        _close(f"dkc[{j}]", from_dev(g["dkc"])[0][j], r["dkc"][j], "bf16")
        _close(f"dvc[{j}]", from_dev(g["dvc"])[0][j], r["dvc"][j], "bf16")
    for rr in (cfg.raw_before, cfg.raw_before + 5000, cfg.R - 1):
        p = cfg.raw_pos0 + rr
        users = np.arange(max(0, p - cfg.pos0), min(cfg.T, p - cfg.pos0 + cfg.W))
        r = ref_over(users)
        _close(f"dkr[{rr}]", from_dev(g["dkr"])[0][rr], r["dkr"][rr], "bf16")
        _close(f"dvr[{rr}]", from_dev(g["dvr"])[0][rr], r["dvr"][rr], "bf16")
    # compressor gradients of the chunk's entries, fed the GPU's entry gradients
    e0, e1 = cfg.n_ctx_entries, cfg.n_cap
    r0, r1 = cfg.raw_before, cfg.raw_before + cfg.n_new_tokens
    for x, dc, dxn, dzn in ((kr, "dkc", "dkr_c", "dz_k"), (vr, "dvc", "dvr_c", "dz_v")):
        rdx, rdz = oracle.compress_backward(x[r0:r1], batch["z"][0], cfg.m,
                                            from_dev(g[dc])[0][e0:e1])
        assert np.max(np.abs(from_dev(g[dxn])[0] - rdx)) <= 1e-5 * max(1.0, np.max(np.abs(rdx)))
        assert np.max(np.abs(from_dev(g[dzn])[0] - rdz)) <= 1e-5 * max(1.0, np.max(np.abs(rdz)))
