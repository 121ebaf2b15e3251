"""Pins of the oracle's backward pass (oracle/backward.py) against things
other than its own formulas: central finite differences of the forward
oracle (the derivative's definition), the translation invariance of the
softmax (key gradients of one query sum to zero), probability mass (value
gradients sum to the upstream gradient), and closed forms of the
compressor's gradient (one-hot weights, m = 1, logits gradients summing to
zero over a block)."""

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _attn_case(rng, T=3, H=2, d=3, N=6, R=5, W=3, k=3):
    q = rng.standard_normal((T, H, d))
    kc = rng.standard_normal((N, d))
    vc = rng.standard_normal((N, d))
    kr = rng.standard_normal((R, d))
    vr = rng.standard_normal((R, d))
    raw_pos0 = 20
    pos = raw_pos0 + R - T + np.arange(T)                  # last T raw rows are the queries
    idx = np.full((T, k), -1, np.int32)
    for t in range(T):
        sel = np.sort(rng.choice(N, size=k - (t % 2), replace=False))   # ragged: -1 padding
        idx[t, :sel.size] = sel
    dout = rng.standard_normal((T, H, d))
    scale = 0.7
    return q, kc, vc, idx, kr, vr, raw_pos0, pos, W, scale, dout


def _loss(args, which=None, value=None):
    q, kc, vc, idx, kr, vr, raw_pos0, pos, W, scale, dout = args
    arrs = {"q": q, "kc": kc, "vc": vc, "kr": kr, "vr": vr}
    if which is not None:
        arrs = dict(arrs)
        arrs[which] = value
    O, _ = oracle.attend(arrs["q"], arrs["kc"], arrs["vc"], idx, arrs["kr"], arrs["vr"], raw_pos0,
                         pos, W, scale)
    return float((O * dout).sum())


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_attend_backward_matches_finite_differences(seed):
    rng = np.random.default_rng(7000 + seed)
    args = _attn_case(rng)
    q, kc, vc, idx, kr, vr, raw_pos0, pos, W, scale, dout = args
    g = oracle.attend_backward(q, kc, vc, idx, kr, vr, raw_pos0, pos, W, scale, dout)
    h = 1e-6
    for name, key in (("q", "dq"), ("kc", "dkc"), ("vc", "dvc"), ("kr", "dkr"), ("vr", "dvr")):
        base = {"q": q, "kc": kc, "vc": vc, "kr": kr, "vr": vr}[name]
        num = np.zeros_like(base)
        for i in np.ndindex(base.shape):
            up, dn = base.copy(), base.copy()
            up[i] += h
            dn[i] -= h
            num[i] = (_loss(args, name, up) - _loss(args, name, dn)) / (2 * h)
        assert np.allclose(g[key], num, rtol=1e-6, atol=1e-8), (name, np.abs(g[key] - num).max())


def test_attend_backward_invariants():
    rng = np.random.default_rng(7100)
    q, kc, vc, idx, kr, vr, raw_pos0, pos, W, scale, dout = _attn_case(rng, T=4, H=3, d=5, N=9,
                                                                      R=7, W=4, k=5)
    g = oracle.attend_backward(q, kc, vc, idx, kr, vr, raw_pos0, pos, W, scale, dout)
    # adding one vector to every key of a query shifts all its logits
    # equally: the key gradients of the whole problem sum to zero
    assert np.allclose(g["dkc"].sum(axis=0) + g["dkr"].sum(axis=0), 0.0, atol=1e-12)
    # probabilities sum to one: value gradients sum to the upstream gradient
    assert np.allclose(g["dvc"].sum(axis=0) + g["dvr"].sum(axis=0), dout.sum(axis=(0, 1)))
    # rows nobody attends get no gradient
    used = np.unique(idx[idx >= 0])
    unused = np.setdiff1d(np.arange(kc.shape[0]), used)
    assert np.all(g["dkc"][unused] == 0) and np.all(g["dvc"][unused] == 0)


def test_attend_backward_single_key_closed_form():
    # one key per query (W = 1, nothing selected): p = 1, so dq = dK = 0
    # and dV = the sum of dout over heads
    rng = np.random.default_rng(7200)
    T, H, d, R = 3, 4, 6, 3
    q = rng.standard_normal((T, H, d))
    kr, vr = rng.standard_normal((R, d)), rng.standard_normal((R, d))
    pos = np.arange(T)
    idx = np.full((T, 2), -1, np.int32)
    dout = rng.standard_normal((T, H, d))
    g = oracle.attend_backward(q, np.zeros((1, d)), np.zeros((1, d)), idx, kr, vr, 0, pos, 1, 0.5,
                               dout)
    assert np.allclose(g["dq"], 0) and np.allclose(g["dkr"], 0)
    assert np.allclose(g["dvr"], dout.sum(axis=1))


def test_hca_backward_is_attend_backward_over_all_entries():
    rng = np.random.default_rng(7300)
    T, H, d, m, N, R, W = 3, 2, 4, 2, 5, 4, 2
    q = rng.standard_normal((T, H, d))
    kc, vc = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    kr, vr = rng.standard_normal((R, d)), rng.standard_normal((R, d))
    pos = np.array([5, 6, 7])
    dout = rng.standard_normal((T, H, d))
    g1 = oracle.hca_attend_backward(q, kc, vc, kr, vr, 4, pos, m, W, 0.3, dout)
    idx = np.stack([np.r_[np.arange(v), -np.ones(N - v, int)] for v in (pos + 1) // m])
    g2 = oracle.attend_backward(q, kc, vc, idx, kr, vr, 4, pos, W, 0.3, dout)
    for key in g1:
        assert np.array_equal(g1[key], g2[key]), key


@pytest.mark.parametrize("m", [1, 3, 4])
def test_compress_backward_matches_finite_differences(m):
    rng = np.random.default_rng(7400 + m)
    nb, d = 3, 4
    x = rng.standard_normal((nb * m, d))
    z = rng.standard_normal((nb * m, d)) * 2
    dc = rng.standard_normal((nb, d))
    dx, dz = oracle.compress_backward(x, z, m, dc)
    h = 1e-6
    loss = lambda xx, zz: float((oracle.compress(xx, zz, m) * dc).sum())
    for arr, g, is_x in ((x, dx, True), (z, dz, False)):
        num = np.zeros_like(arr)
        for i in np.ndindex(arr.shape):
            up, dn = arr.copy(), arr.copy()
            up[i] += h
            dn[i] -= h
            num[i] = ((loss(up, z) - loss(dn, z)) if is_x else (loss(x, up) - loss(x, dn))) / (2 * h)
        assert np.allclose(g, num, rtol=1e-6, atol=1e-8)


def test_compress_backward_closed_forms():
    rng = np.random.default_rng(7500)
    nb, m, d = 4, 4, 5
    x = rng.standard_normal((nb * m, d))
    dc = rng.standard_normal((nb, d))
    # logits gradients of a block sum to zero (softmax)
    z = rng.standard_normal((nb * m, d))
    _, dz = oracle.compress_backward(x, z, m, dc)
    assert np.allclose(dz.reshape(nb, m, d).sum(axis=1), 0.0, atol=1e-12)
    # one-hot weights: the gradient goes to the picked token only
    pick = rng.integers(0, m, size=(nb, d))
    z1 = np.full((nb, m, d), -1e30)
    np.put_along_axis(z1, pick[:, None, :], 0.0, axis=1)
    dx, dz = oracle.compress_backward(x, z1.reshape(nb * m, d), m, dc)
    want = np.zeros((nb, m, d))
    np.put_along_axis(want, pick[:, None, :], dc[:, None, :], axis=1)
    assert np.array_equal(dx, want.reshape(nb * m, d))
    assert np.all(dz == 0)
    # m = 1: the identity
    dx, dz = oracle.compress_backward(x[:nb], z[:nb], 1, dc)
    assert np.array_equal(dx, dc) and np.all(dz == 0)
