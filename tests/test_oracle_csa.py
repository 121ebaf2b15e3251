"""Pins of the CSA / HCA oracle: hand-worked fixtures, closed forms, special
cases that reduce to a library routine (NumPy matmul, PyTorch's
scaled_dot_product_attention in float64), brute force on tiny inputs and
invariants.  None of these re-types the oracle's own formula."""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import (attend, compress, csa_forward, hca_attend, indexer_scores,
                    topk_select, visible_count)


# ----------------------------------------------------------------- compress

def test_compress_golden(load_golden):
    g = load_golden("compress_two_blocks.json")
    got = compress(np.array(g["x"], float), np.array(g["logits"], float), g["m"])
    assert np.allclose(got, g["expected"], rtol=0, atol=g["tol"])


def test_compress_one_hot_logits_subsample_tokens():
    rng = np.random.default_rng(0)
    m, nb, d = 4, 37, 16
    x = rng.standard_normal((nb * m, d))
    pick = rng.integers(0, m, size=(nb, d))
    z = np.full((nb, m, d), -1e30)
    np.put_along_axis(z, pick[:, None, :], 0.0, axis=1)
    got = compress(x, z.reshape(nb * m, d), m)
    want = np.take_along_axis(x.reshape(nb, m, d), pick[:, None, :], axis=1)[:, 0]
    assert np.array_equal(got, want)


def test_compress_equal_logits_is_block_mean_and_m1_is_identity():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((64, 8))
    z = np.tile(rng.standard_normal((16, 1, 8)), (1, 4, 1)).reshape(64, 8)
    got = compress(x, z, 4)
    assert np.allclose(got, x.reshape(16, 4, 8).mean(axis=1), atol=1e-14)
    assert np.array_equal(compress(x, rng.standard_normal((64, 8)), 1), x)


def test_compress_chunked_equals_whole_and_shift_invariance():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((128, 8))
    z = rng.standard_normal((128, 8))
    whole = compress(x, z, 4)
    parts = np.concatenate([compress(x[:48], z[:48], 4), compress(x[48:], z[48:], 4)])
    assert np.array_equal(whole, parts)
    # adding a constant per (block, channel) to the logits leaves the
    # weights unchanged; a softmax taken over the wrong axis would not
    c = np.repeat(rng.standard_normal((32, 8)) * 5, 4, axis=0)
    assert np.allclose(compress(x, z + c, 4), whole, atol=1e-13)
    # weights are a convex combination: every entry lies in its block's range
    xb = x.reshape(32, 4, 8)
    assert np.all(whole <= xb.max(axis=1) + 1e-12) and np.all(whole >= xb.min(axis=1) - 1e-12)


def test_compress_rejects_partial_block():
    with pytest.raises(AssertionError):
        compress(np.zeros((6, 2)), np.zeros((6, 2)), 4)


# ------------------------------------------------------------------ indexer

def test_visible_count():
    assert list(visible_count(np.arange(9), 4)) == [0, 0, 0, 1, 1, 1, 1, 2, 2]
    assert list(visible_count(np.arange(4), 1)) == [1, 2, 3, 4]
    assert visible_count(131072, 4) == 32768 and visible_count(1048576, 128) == 8192


def test_indexer_golden(load_golden):
    g = load_golden("indexer_two_heads.json")
    T = len(g["pos"])
    qi = np.tile(np.array(g["qi"], float)[None], (T, 1, 1))
    w = np.tile(np.array(g["w"], float)[None], (T, 1))
    for act, key in (("relu", "expected_relu"), ("identity", "expected_identity")):
        S = indexer_scores(qi, w, np.array(g["ki"], float), g["pos"], g["m"], act)
        want = np.array([[np.nan if v is None else v for v in row] for row in g[key]])
        assert np.array_equal(np.isnan(S), np.isnan(want))
        assert np.allclose(S[~np.isnan(S)], want[~np.isnan(want)], atol=1e-14)


def test_indexer_single_head_identity_is_matmul():
    rng = np.random.default_rng(4)
    T, N, d = 9, 20, 16
    qi = rng.standard_normal((T, 1, d))
    ki = rng.standard_normal((N, d))
    pos = np.arange(20, 20 + T)
    S = indexer_scores(qi, np.ones((T, 1)), ki, pos, 2, "identity")
    full = np.matmul(qi[:, 0, :], ki.T)
    V = visible_count(pos, 2)
    for t in range(T):
        assert np.allclose(S[t, :V[t]], full[t, :V[t]], rtol=1e-13, atol=1e-13)
        assert np.all(np.isnan(S[t, V[t]:]))


def test_indexer_relu_properties():
    rng = np.random.default_rng(5)
    T, H, N, d = 6, 8, 30, 12
    qi = rng.standard_normal((T, H, d))
    w = rng.random((T, H))
    ki = rng.standard_normal((N, d))
    pos = np.full(T, 4 * N - 1)
    S = indexer_scores(qi, w, ki, pos, 4, "relu")
    assert np.all(S >= 0)
    # homogeneous in the head weights
    assert np.allclose(indexer_scores(qi, 2.5 * w, ki, pos, 4), 2.5 * S, rtol=1e-13)
    # a head whose dot products are all negative contributes nothing
    ki_pos = np.abs(ki)
    qi2 = qi.copy()
    qi2[:, 0, :] = -np.abs(qi2[:, 0, :])
    S_with = indexer_scores(qi2, w, ki_pos, pos, 4)
    w0 = w.copy()
    w0[:, 0] = 0
    assert np.allclose(S_with, indexer_scores(qi2, w0, ki_pos, pos, 4), rtol=1e-13)
    # with every dot product positive, ReLU and identity agree
    qi3 = np.abs(qi)
    assert np.allclose(indexer_scores(qi3, w, ki_pos, pos, 4, "relu"),
                       indexer_scores(qi3, w, ki_pos, pos, 4, "identity"), rtol=1e-13)


# -------------------------------------------------------------------- top-k

def test_topk_golden(load_golden):
    g = load_golden("topk_ties.json")
    for c in g["cases"]:
        s = np.array([float(v) for v in c["scores"]])
        assert list(topk_select(s, c["visible"], c["k"])) == c["expected"]


def test_topk_matches_brute_force_sort():
    rng = np.random.default_rng(6)
    for trial in range(300):
        n = int(rng.integers(0, 40))
        v = int(rng.integers(0, n + 1))
        k = int(rng.integers(1, 45))
        s = rng.integers(-3, 4, size=n).astype(float)  # many ties
        if trial % 3 == 0:
            s = rng.standard_normal(n)
        ranked = sorted(range(v), key=lambda j: (-s[j], j))
        want = sorted(ranked[:k]) + [-1] * (k - min(k, v))
        assert list(topk_select(s, v, k)) == want


def test_topk_rejects_nonfinite():
    with pytest.raises(AssertionError):
        topk_select(np.array([1.0, np.nan]), 2, 1)


# ---------------------------------------------------------------- attention

def _sdpa(q, keys, vals, mask, scale):
    """float64 scaled_dot_product_attention with a boolean keep-mask.
    q [T, H, d], keys/vals [L, d], mask [T, L]."""
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]           # [1, H, T, d]
    kt = torch.from_numpy(keys)[None, None].expand(1, q.shape[1], -1, -1)
    vt = torch.from_numpy(vals)[None, None].expand(1, q.shape[1], -1, -1)
    m = torch.from_numpy(mask)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    return o[0].permute(1, 0, 2).numpy()


def test_attend_golden(load_golden):
    g = load_golden("attend_two_keys.json")
    O, lse = attend(np.array(g["q"]), np.array(g["kc"]), np.array(g["vc"]),
                    np.array(g["idx"]), np.array(g["kr"]), np.array(g["vr"]),
                    g["raw_pos0"], g["pos"], g["W"], g["scale"])
    assert np.allclose(O, g["expected_out"], atol=g["tol"])
    assert np.allclose(lse, g["expected_lse"], atol=g["tol"])


def test_m1_full_k_is_dense_causal_attention_plus_window():
    """With m = 1 every raw token is its own entry; with k >= V(t) the CSA
    output equals dense causal attention over tokens 0..t together with a
    second copy of the window tokens."""
    rng = np.random.default_rng(8)
    n, d, H, HI, W = 40, 8, 3, 2, 5
    K = rng.standard_normal((n, d))
    V = rng.standard_normal((n, d))
    Z = rng.standard_normal((n, d))
    qi = rng.standard_normal((n, HI, d))
    w = rng.random((n, HI))
    q = rng.standard_normal((n, H, d))
    scale = 1 / math.sqrt(d)
    res = csa_forward(K, V, Z, qi, w, q, 1, n, W, scale)
    t = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    mask = np.concatenate([j <= t, (j <= t) & (j > t - W)], axis=1)
    want = _sdpa(q, np.concatenate([K, K]), np.concatenate([V, V]), mask, scale)
    assert np.allclose(res["out"], want, atol=1e-12)


def test_short_prefix_is_pure_sliding_window_and_t0_is_v0():
    rng = np.random.default_rng(9)
    m, n, d, H, W = 8, 7, 4, 2, 3   # t < m-1: nothing compressed yet
    K = rng.standard_normal((n, d))
    V = rng.standard_normal((n, d))
    q = rng.standard_normal((n, H, d))
    idx = np.full((n, 4), -1)
    O, _ = attend(q, np.zeros((0, d)), np.zeros((0, d)), idx, K, V, 0, np.arange(n), W, 0.5)
    t = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    want = _sdpa(q, K, V, (j <= t) & (j > t - W), 0.5)
    assert np.allclose(O, want, atol=1e-12)
    assert np.array_equal(O[0], np.tile(V[0], (H, 1)))


def test_attend_matches_sdpa_on_explicit_key_lists():
    rng = np.random.default_rng(10)
    N, R, d, H, W, T = 50, 30, 16, 4, 6, 5
    kc, vc = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    kr, vr = rng.standard_normal((R, d)), rng.standard_normal((R, d))
    raw_pos0 = 200
    pos = raw_pos0 + np.array([5, 9, 17, 25, 29])
    q = rng.standard_normal((T, H, d))
    idx = np.full((T, 12), -1)
    for i in range(T):
        c = rng.choice(N, size=int(rng.integers(0, 12)), replace=False)
        idx[i, :c.size] = np.sort(c)
    O, lse = attend(q, kc, vc, idx, kr, vr, raw_pos0, pos, W, 0.3)
    for i in range(T):
        sel = idx[i][idx[i] >= 0]
        p = np.arange(max(0, pos[i] - W + 1), pos[i] + 1) - raw_pos0
        keys = np.concatenate([kc[sel], kr[p]])
        vals = np.concatenate([vc[sel], vr[p]])
        want = _sdpa(q[i:i + 1], keys, vals, np.ones((1, len(keys)), bool), 0.3)
        assert np.allclose(O[i:i + 1], want, atol=1e-12)
        lg = torch.from_numpy(q[i] @ keys.T * 0.3)
        assert np.allclose(lse[i], torch.logsumexp(lg, dim=1).numpy(), atol=1e-12)


def test_attend_invariants_permutation_and_lse_merge():
    rng = np.random.default_rng(12)
    N, d, H, W = 40, 8, 2, 4
    kc, vc = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    kr, vr = rng.standard_normal((10, d)), rng.standard_normal((10, d))
    q = rng.standard_normal((1, H, d))
    pos = np.array([9])
    sel = rng.choice(N, size=16, replace=False)
    O, lse = attend(q, kc, vc, sel[None], kr, vr, 0, pos, W, 0.4)
    O2, lse2 = attend(q, kc, vc, rng.permutation(sel)[None], kr, vr, 0, pos, W, 0.4)
    assert np.allclose(O, O2, atol=1e-13) and np.allclose(lse, lse2, atol=1e-13)
    # split: entries A (no window) and entries B (+ window), merged by LSE
    A, Bs = sel[:7], sel[7:]
    OA, lA = attend(q, kc, vc, A[None], kr, vr, 0, pos, 0, 0.4)
    OB, lB = attend(q, kc, vc, Bs[None], kr, vr, 0, pos, W, 0.4)
    mx = np.maximum(lA, lB)
    wa, wb = np.exp(lA - mx), np.exp(lB - mx)
    merged = (wa[..., None] * OA + wb[..., None] * OB) / (wa + wb)[..., None]
    assert np.allclose(merged, O, atol=1e-13)
    assert np.allclose(mx + np.log(wa + wb), lse, atol=1e-13)


def test_zero_scale_gives_mean_of_values():
    rng = np.random.default_rng(13)
    kc, vc = rng.standard_normal((10, 4)), rng.standard_normal((10, 4))
    kr, vr = rng.standard_normal((5, 4)), rng.standard_normal((5, 4))
    idx = np.array([[1, 4, 7, -1]])
    O, lse = attend(rng.standard_normal((1, 3, 4)), kc, vc, idx, kr, vr, 0, [4], 2, 0.0)
    want = np.concatenate([vc[[1, 4, 7]], vr[[3, 4]]]).mean(axis=0)
    assert np.allclose(O[0], want, atol=1e-14)
    assert np.allclose(lse, math.log(5), atol=1e-14)


def test_full_k_selection_equals_hca():
    """k >= V(t): the top-k keeps every visible entry, so CSA attention is
    HCA-style dense attention over the compressed cache."""
    rng = np.random.default_rng(14)
    m, N, d, H, HI, W, T = 4, 12, 8, 3, 2, 4, 6
    kc, vc = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    kr, vr = rng.standard_normal((20, d)), rng.standard_normal((20, d))
    raw_pos0 = 30
    pos = raw_pos0 + np.arange(14, 20)
    q = rng.standard_normal((T, H, d))
    qi, w = rng.standard_normal((T, HI, d)), rng.random((T, HI))
    S = indexer_scores(qi, w, kc, pos, m)
    Vt = visible_count(pos, m)
    idx = np.stack([topk_select(S[t], int(Vt[t]), 64) for t in range(T)])
    O, lse = attend(q, kc, vc, idx, kr, vr, raw_pos0, pos, W, 0.35)
    Oh, lseh = hca_attend(q, kc, vc, kr, vr, raw_pos0, pos, m, W, 0.35)
    assert np.allclose(O, Oh, atol=1e-13) and np.allclose(lse, lseh, atol=1e-13)


def test_causality_of_selection():
    """No compressed block that ends after the query position is ever
    selectable, whatever its score."""
    rng = np.random.default_rng(15)
    m, n, d = 4, 64, 8
    res = csa_forward(rng.standard_normal((n, d)), rng.standard_normal((n, d)),
                      rng.standard_normal((n, d)), rng.standard_normal((n, 2, d)),
                      rng.random((n, 2)), rng.standard_normal((n, 2, d)), m, 5, 8, 0.3)
    for t in range(n):
        sel = res["idx"][t][res["idx"][t] >= 0]
        assert np.all((sel + 1) * m - 1 <= t)
        assert len(sel) == min(5, (t + 1) // m)
        assert np.all(np.diff(sel) > 0)
