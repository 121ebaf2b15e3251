"""Seeded sweep of small random configurations through the whole path
(compress, indexer + top-k, attention; HCA and window-only layers; the
fused block-boundary selection; the backward), each checked against the
oracle: scores to 1e-3 relative, indices bit-exact on the GPU's scores,
outputs and gradients to the dtype's tolerance.  Shapes are drawn so that
tiles, chunks and splits end raggedly; positions include the first tokens
(empty or partial windows, no visible entries)."""

import numpy as np
import pytest
import torch

from conftest import ensure_library
from gpu_util import decode, from_dev, rel_l2, say, score_close, to_dev

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


def _draw(seed):
    r = np.random.default_rng(9000 + seed)
    storage = ["f32", "bf16"][seed % 2]
    d = int(r.choice([64, 128]))
    H = int(r.choice([1, 7, 16, 33, 64]))
    m = int(r.choice([1, 2, 4, 8]))
    T = int(r.choice([1, 1, 3, 9, 17]))
    n_ctx = int(r.integers(0, 700))
    W = int(r.choice([0, 1, 5, 32, 128]))
    k = int(r.choice([1, 7, 64, 300]))
    kind = r.choice(["csa", "csa", "csa", "hca", "swa"])
    if kind == "swa" and W == 0:
        W = 4
    pos0 = int(r.integers(0, m * n_ctx + 2)) if n_ctx else int(r.integers(0, 6))
    H_I = int(r.choice([1, 4, 64]))
    return dict(storage=storage, d=d, H=H, m=m, T=T, n_ctx=n_ctx, W=W, k=k, kind=kind,
                pos0=pos0, H_I=H_I, B=int(r.choice([1, 3])))


@pytest.mark.parametrize("seed", range(48))
def test_random_configuration(seed):
    c = _draw(seed)
    say("sweep", seed, c)
    n_new = c["T"] if c["T"] % c["m"] == 0 and c["pos0"] % c["m"] == 0 and c["T"] > 1 else 0
    hca, swa = c["kind"] == "hca", c["kind"] == "swa"
    cfg = WL.Workload(
        name=f"sweep{seed}", number=900 + seed, B=c["B"], T=c["T"], pos0=c["pos0"], m=c["m"],
        d=c["d"], H=c["H"], W=c["W"], n_ctx_entries=max(1, c["n_ctx"]), n_new_tokens=n_new,
        raw_before=c["W"] + 1, H_I=0 if (hca or swa) else c["H_I"],
        d_I=0 if (hca or swa) else c["d"], k=0 if (hca or swa) else c["k"],
        storage=c["storage"], swa=swa)
    # positions of the new tokens continue the context when compressing;
    # otherwise every query's visible entries stay within the cache
    if n_new:
        cfg = cfg.replace(pos0=cfg.n_ctx_entries * cfg.m)
    else:
        cfg = cfg.replace(pos0=max(0, min(cfg.pos0, cfg.m * cfg.n_cap - cfg.T)))
    batch = WL.make_batch(cfg)
    step = CSAStep(cfg, batch)
    step.run()
    torch.cuda.synchronize()
    tol_o = 1e-4 if cfg.storage == "f32" else 2e-2
    for b in range(cfg.B):
        pos = cfg.pos0 + np.arange(cfg.T)
        kc = decode(from_dev(step.kc)[b])
        vc = decode(from_dev(step.vc)[b])
        if n_new:
            x = decode(batch["kr"][b][cfg.raw_before:cfg.raw_before + n_new])
            ref = oracle.compress(x, batch["z"][b], cfg.m)
            got = kc[cfg.n_ctx_entries:cfg.n_cap]
            assert np.max(np.abs(got - ref)) <= (1e-5 if cfg.storage == "f32" else 2e-2)
        q, kr, vr = decode(batch["q"][b]), decode(batch["kr"][b]), decode(batch["vr"][b])
        if hca:
            ref_o, ref_l = oracle.hca_attend(q, kc, vc, kr, vr, cfg.raw_pos0, pos, cfg.m, cfg.W,
                                             cfg.scale)
            idx = oracle.hca_indices(pos, cfg.m)
            idx = np.where(idx < cfg.n_cap, idx, -1)
        elif swa:
            idx = np.zeros((cfg.T, 0), np.int32)
            ref_o, ref_l = oracle.attend(q, kc, vc, idx, kr, vr, cfg.raw_pos0, pos, cfg.W,
                                         cfg.scale)
        else:
            V = np.minimum(oracle.visible_count(pos, cfg.m), cfg.n_cap)
            sc = from_dev(step.scores)[b]
            ref_s = oracle.indexer_scores(decode(batch["qi"][b]), batch["w"][b], kc, pos, cfg.m)
            idx = from_dev(step.idx)[b]
            for i in range(cfg.T):
                assert score_close(sc[i, :V[i]], ref_s[i, :V[i]]) <= 1.0
                want = oracle.topk_select(sc[i, :V[i]].astype(np.float64), int(V[i]), cfg.k)
                assert np.array_equal(idx[i], want), (b, i)
            ref_o, ref_l = oracle.attend(q, kc, vc, idx, kr, vr, cfg.raw_pos0, pos, cfg.W,
                                         cfg.scale)
        out = from_dev(step.out)[b]
        lse = from_dev(step.lse)[b]
        has_keys = np.isfinite(ref_l)
        assert np.max(np.abs(out - ref_o)) <= tol_o, np.max(np.abs(out - ref_o))
        assert np.allclose(lse[has_keys], ref_l[has_keys], atol=1e-3, rtol=1e-4)
        assert np.all(np.isinf(lse[~has_keys]))
    # the backward of the same attention (CSA / window-only with an index list)
    if not hca and cfg.d in (64, 128) and cfg.k <= 4096:
        rng = np.random.default_rng(9500 + seed)
        dout = rng.standard_normal(tuple(step.out.shape)).astype(np.float32)
        idx_d = step.idx if not swa else torch.full((cfg.B, cfg.T, 1), -1, dtype=torch.int32,
                                                     device=step.out.device)
        g = csa.csa_attend_backward(step.q, step.kc, step.vc, idx_d, step.kr, step.vr,
                                    step.raw_pos0, step.pos0, cfg.W, cfg.scale, step.out,
                                    step.lse, to_dev(dout))
        torch.cuda.synchronize()
        for b in range(cfg.B):
            pos = cfg.pos0 + np.arange(cfg.T)
            ref = oracle.attend_backward(decode(batch["q"][b]), decode(from_dev(step.kc)[b]),
                                         decode(from_dev(step.vc)[b]), from_dev(idx_d)[b],
                                         decode(batch["kr"][b]), decode(batch["vr"][b]),
                                         cfg.raw_pos0, pos, cfg.W, cfg.scale, dout[b])
            # errors are measured against the size of the terms that cancel
            # (a query with a single key has dq = dK = 0 exactly, which fp32
            # reaches only up to rounding): scale |k| |dout| |v| for dq / dK,
            # |dout| for dV
            amax = lambda a: float(np.max(np.abs(a))) if a.size else 0.0
            kv = max(amax(decode(from_dev(step.kc)[b])), amax(decode(batch["kr"][b])),
                     amax(decode(batch["q"][b])))
            vv = max(amax(decode(from_dev(step.vc)[b])), amax(decode(batch["vr"][b])))
            terms = {"dq": cfg.scale * kv * amax(dout[b]) * vv, "dkc": cfg.scale * kv * amax(dout[b]) * vv,
                     "dkr": cfg.scale * kv * amax(dout[b]) * vv, "dvc": amax(dout[b]),
                     "dvr": amax(dout[b])}
            for key in ("dq", "dkc", "dvc") + (("dkr", "dvr") if cfg.W else ()):
                got = from_dev(g[key])[b]
                scale = max(amax(ref[key]), terms[key], 1e-30)
                err = float(np.max(np.abs(got - ref[key]))) / scale
                assert err <= (1e-5 if cfg.storage == "f32" else 1e-2), (key, err)
