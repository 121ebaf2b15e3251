"""A sequence's results do not depend on where it sits in the batch
("DeepSeek V4 technical review", takeshell.com, section 6.2 Deterministic
Training: the same token gives bitwise-identical output whatever its
position in the batch, with no atomic-add nondeterminism).

Each case runs a batch, then the same sequences in another order, and
compares every per-sequence result bit for bit: indexer scores, top-k
lists, attention output and log-sum-exp, and the backward pass's
gradients (dq and the per-sequence key / value gradients, which are sums
over the sequence's own query rows)."""

import numpy as np
import pytest
import torch

from conftest import ensure_library
from gpu_util import bf16_codes, say, to_dev

pytestmark = pytest.mark.gpu

ensure_library()
import long_context_sparse_16_amd as csa  # noqa: E402


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _perm(t: torch.Tensor, perm) -> torch.Tensor:
    return t[torch.as_tensor(perm, device=t.device)].contiguous()


def _same(name, a: torch.Tensor, b: torch.Tensor) -> None:
    assert a.shape == b.shape, (name, a.shape, b.shape)
    assert torch.equal(a, b), (name, "differs after reordering the batch")


def _decode_inputs(rng, B, n_cap, H_I, d_I, H, d, W, m):
    R = W + 7
    kc = to_dev(bf16_codes(rng.standard_normal((B, n_cap, d))))
    vc = to_dev(bf16_codes(rng.standard_normal((B, n_cap, d))))
    kr = to_dev(bf16_codes(rng.standard_normal((B, R, d))))
    vr = to_dev(bf16_codes(rng.standard_normal((B, R, d))))
    q = to_dev(bf16_codes(rng.standard_normal((B, 1, H, d))))
    qi = to_dev(bf16_codes(rng.standard_normal((B, 1, H_I, d_I))))
    w = to_dev(rng.random((B, 1, H_I), dtype=np.float32))
    # positions spread over the cache; some sequences see only part of it
    pos0 = np.sort(rng.integers(m * n_cap // 4, m * n_cap, size=B)).astype(np.int64)
    pos0[-1] = m * n_cap - 1
    raw_pos0 = pos0 - R + 1
    return dict(q=q, kc=kc, vc=vc, kr=kr, vr=vr, qi=qi, w=w, pos0=to_dev(pos0),
                raw_pos0=to_dev(raw_pos0))


def _csa_decode(x, m, k, W, ki):
    scores, idx = csa.csa_index_topk(x["qi"], x["w"], ki, x["pos0"], m, k)
    scale = 1.0 / np.sqrt(x["q"].shape[-1])
    out, lse = csa.csa_attend(x["q"], x["kc"], x["vc"], idx, x["kr"], x["vr"], x["raw_pos0"],
                              x["pos0"], W, scale)
    return dict(scores=scores, idx=idx, out=out, lse=lse)


@pytest.mark.parametrize("n_cap", [3000, 9000])   # top-k row path / split path
def test_csa_decode_batch_position(n_cap):
    say("batch position: csa decode", n_cap)
    rng = np.random.default_rng(9100 + n_cap)
    B, H_I, d_I, H, d, W, m, k = 6, 16, 128, 64, 128, 64, 4, 256
    x = _decode_inputs(rng, B, n_cap, H_I, d_I, H, d, W, m)
    a = _csa_decode(x, m, k, W, x["kc"])
    perm = [4, 1, 5, 0, 3, 2]
    xp = {key: _perm(v, perm) for key, v in x.items()}
    b = _csa_decode(xp, m, k, W, xp["kc"])
    torch.cuda.synchronize()
    for key in ("idx", "out", "lse"):
        _same(key, _perm(a[key], perm), b[key])
    # scores: only the entries a query can see are written
    pos = x["pos0"].cpu().numpy()
    for j, src in enumerate(perm):
        V = int(min(n_cap, (pos[src] + 1) // m))
        _same(f"scores[{src}]", a["scores"][src, 0, :V], b["scores"][j, 0, :V])


def test_csa_decode_batch_size():
    """A sequence decoded alone (B = 1) and inside a batch of 6: the scores
    and top-k lists are bit-identical (every score is a fixed-order sum of
    its own row), while the attention output and lse may differ in the last
    bits, because the number of key splits -- and so the order of the merge's
    fp32 sums -- follows the batch's query rows (B*T)."""
    say("batch size: csa decode")
    rng = np.random.default_rng(9150)
    B, n_cap, H_I, d_I, H, d, W, m, k = 6, 9000, 16, 128, 64, 128, 64, 4, 256
    x = _decode_inputs(rng, B, n_cap, H_I, d_I, H, d, W, m)
    a = _csa_decode(x, m, k, W, x["kc"])
    pos = x["pos0"].cpu().numpy()
    for src in (0, 3, 5):
        one = {key: v[src:src + 1].contiguous() for key, v in x.items()}
        b = _csa_decode(one, m, k, W, one["kc"])
        torch.cuda.synchronize()
        V = int(min(n_cap, (pos[src] + 1) // m))
        _same(f"scores[{src}]", a["scores"][src, 0, :V], b["scores"][0, 0, :V])
        _same(f"idx[{src}]", a["idx"][src:src + 1], b["idx"])
        for key, tol in (("out", 1e-5), ("lse", 1e-6)):
            ref = a[key][src:src + 1].double()
            err = float((b[key].double() - ref).abs().max() / ref.abs().max())
            say("  ", key, src, "max rel diff", err)
            assert err <= tol, (key, src, err)


def test_hca_decode_batch_position():
    say("batch position: hca decode")
    rng = np.random.default_rng(9200)
    B, n_cap, H, d, W, m = 5, 700, 64, 128, 128, 128
    x = _decode_inputs(rng, B, n_cap, 4, 128, H, d, W, m)
    scale = 1.0 / np.sqrt(d)

    def run(y):
        out, lse = csa.hca_attend(y["q"], y["kc"], y["vc"], m, y["kr"], y["vr"], y["raw_pos0"],
                                  y["pos0"], W, scale)
        return dict(out=out, lse=lse)

    a = run(x)
    perm = [2, 4, 0, 3, 1]
    b = run({key: _perm(v, perm) for key, v in x.items()})
    torch.cuda.synchronize()
    for key in a:
        _same(key, _perm(a[key], perm), b[key])


@pytest.mark.parametrize("storage", ["f32", "bf16"])
def test_prefill_forward_backward_batch_position(storage):
    """Several query rows per sequence, so the key / value gradients are
    sums over rows (the deterministic per-entry and per-raw-row sums)."""
    say("batch position: prefill forward + backward", storage)
    rng = np.random.default_rng(9300 + len(storage))
    B, T, H, d, n_cap, k, W, m = 3, 45, 64, 128, 400, 48, 16, 4
    R = T + W

    def store(a):
        return a.astype(np.float32) if storage == "f32" else bf16_codes(a)

    q = store(rng.standard_normal((B, T, H, d)))
    kc = store(rng.standard_normal((B, n_cap, d)))
    vc = store(rng.standard_normal((B, n_cap, d)))
    kr = store(rng.standard_normal((B, R, d)))
    vr = store(rng.standard_normal((B, R, d)))
    pos0 = np.array([3, 700, 4 * n_cap - T], np.int64)
    raw_pos0 = pos0 + T - R
    idx = np.full((B, T, k), -1, np.int32)
    for b in range(B):
        for i in range(T):
            V = int(min(n_cap, (pos0[b] + i + 1) // m))
            n = min(k, V) - (i % 4 == 2 and min(k, V) > 0)
            if n > 0:
                idx[b, i, :n] = np.sort(rng.choice(V, size=n, replace=False))
    dout = rng.standard_normal((B, T, H, d)).astype(np.float32)
    x = dict(q=to_dev(q), kc=to_dev(kc), vc=to_dev(vc), idx=to_dev(idx), kr=to_dev(kr),
             vr=to_dev(vr), raw_pos0=to_dev(raw_pos0), pos0=to_dev(pos0), dout=to_dev(dout))
    scale = 1.0 / np.sqrt(d)

    def run(y):
        args = (y["q"], y["kc"], y["vc"], y["idx"], y["kr"], y["vr"], y["raw_pos0"], y["pos0"],
                W, scale)
        out, lse = csa.csa_attend(*args)
        g = csa.csa_attend_backward(*args, out, lse, y["dout"])
        return dict(out=out, lse=lse, **g)

    a = run(x)
    perm = [2, 0, 1]
    b = run({key: _perm(v, perm) for key, v in x.items()})
    torch.cuda.synchronize()
    for key in a:
        _same(key, _perm(a[key], perm), b[key])
