"""Stage-wise parity of the HIP kernels against the fp64 oracle, at sizes the
oracle finishes in seconds that still span several tiles / workgroups and a
ragged tail.  Every call goes through the C ABI (via the ctypes binding)."""

import math

import numpy as np
import pytest
import torch

from conftest import ensure_library
from gpu_util import (DEV, bf16_codes, compress_bound, decode, from_dev, rel_l2, say,
                      score_close, to_dev)

import oracle

pytestmark = pytest.mark.gpu

ensure_library()
import long_context_sparse_16_amd as csa  # noqa: E402


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _store(x, storage):
    return x.astype(np.float32) if storage == "f32" else bf16_codes(x)


# ------------------------------------------------------------- fp8 quantizer

@pytest.mark.parametrize("storage", ["f32", "bf16"])
def test_quantize_fp8_rows_bitexact(storage):
    say("quantize", storage)
    rng = np.random.default_rng(100)
    x = rng.standard_normal((997, 128)).astype(np.float32) * 3
    x[0] = 0.0                                  # zero row -> scale 1
    x[1] = rng.standard_normal(128) * 1e-30     # tiny values: subnormal codes
    x[2, :] = 1.0
    x[2, 7] = -448.0                            # exact scale 1
    # values whose quotient lands on exact e4m3 midpoints (ties to even)
    mids = (oracle.e4m3_decode(np.arange(0x7e)) + oracle.e4m3_decode(np.arange(1, 0x7f))) / 2
    x[3, :] = 0.0
    x[3, :100] = mids[:100]
    x[3, 100] = 448.0
    xs = _store(x, storage)
    codes, scales = csa.csa_quantize_fp8_rows(to_dev(xs))
    torch.cuda.synchronize()
    ref_codes, ref_scales = oracle.quantize_fp8_rows(decode(xs).astype(np.float32))
    assert np.array_equal(from_dev(scales), ref_scales)
    assert np.array_equal(from_dev(codes), ref_codes)


# ----------------------------------------------------------- MXFP4 quantizer

@pytest.mark.parametrize("storage,d", [("f32", 128), ("bf16", 128), ("f32", 96), ("bf16", 256)])
def test_quantize_mxfp4_rows_bitexact(storage, d):
    say("quantize mxfp4", storage, d)
    rng = np.random.default_rng(110 + d)
    x = rng.standard_normal((613, d)).astype(np.float32) * np.exp(rng.uniform(-30, 30, (613, 1)))
    x = x.astype(np.float32)
    x[0] = 0.0                                   # zero blocks -> scale code 0
    x[1, :32] = -0.0
    # exact E2M1 midpoints times the block scale (ties to even) with the
    # block maximum fixing the scale at 2^0 and at 2^-5
    vals = oracle.e2m1_decode(np.arange(8))
    mids = (vals[:-1] + vals[1:]) / 2
    for r, sc in ((2, 1.0), (3, 2.0 ** -5)):
        x[r] = 0.0
        x[r, 0] = 6.0 * sc
        x[r, 1:8] = mids * sc
        x[r, 8:15] = -mids * sc
        x[r, 15] = 7.9 * sc                      # saturates to 6
    x[4, :32] = np.float32(2.0 ** -149)          # smallest subnormal block
    xs = _store(x, storage)
    codes, scales = csa.csa_quantize_mxfp4_rows(to_dev(xs))
    torch.cuda.synchronize()
    ref_codes, ref_scales = oracle.quantize_mxfp4_rows(decode(xs).astype(np.float32))
    assert np.array_equal(from_dev(scales), ref_scales)
    assert np.array_equal(from_dev(codes), ref_codes)


# ---------------------------------------------------------------- compressor

@pytest.mark.parametrize("storage", ["f32", "bf16"])
@pytest.mark.parametrize("m,d,nb", [(4, 64, 37), (4, 128, 600), (128, 128, 5), (1, 64, 9)])
def test_compress_parity(storage, m, d, nb):
    say("compress", storage, m, d, nb)
    rng = np.random.default_rng(200 + m + d)
    B, first, extra = 2, 5, 3
    n_tok = nb * m
    n_cap = first + nb + extra
    x = _store(rng.standard_normal((B, n_tok, d)), storage)
    z = (rng.standard_normal((B, n_tok, d)) * 2).astype(np.float32)
    sentinel = np.full((B, n_cap, d), 7.0, np.float32)
    cache = to_dev(_store(sentinel, storage))
    csa.csa_compress(to_dev(x), to_dev(z), cache, m, first)
    got = decode(from_dev(cache))
    for b in range(B):
        xv = decode(x[b])
        ref = oracle.compress(xv, z[b], m)
        g = got[b, first:first + nb]
        if storage == "f32":
            assert np.max(np.abs(g - ref)) <= 1e-5 * max(1.0, np.max(np.abs(ref)))
        else:
            assert np.all(np.abs(g - ref) <= compress_bound(ref, xv.reshape(nb, m, d), m))
        assert np.all(got[b, :first] == 7.0) and np.all(got[b, first + nb:] == 7.0)


@pytest.mark.parametrize("storage", ["f32", "bf16"])
def test_compress_one_hot_and_chunked_append(storage):
    say("compress one-hot / chunked", storage)
    rng = np.random.default_rng(300)
    B, m, d, nb = 3, 4, 128, 50
    x = _store(rng.standard_normal((B, nb * m, d)), storage)
    pick = rng.integers(0, m, size=(B, nb, d))
    z = np.full((B, nb, m, d), -1e30, np.float32)
    np.put_along_axis(z, pick[:, :, None, :], 0.0, axis=2)
    z = z.reshape(B, nb * m, d)
    cache = to_dev(_store(np.zeros((B, nb, d)), storage))
    csa.csa_compress(to_dev(x), to_dev(z), cache, m, 0)
    got = from_dev(cache)
    want = np.take_along_axis(x.reshape(B, nb, m, d), pick[:, :, None, :], axis=2)[:, :, 0]
    assert np.array_equal(got, want)  # exact subsampling, bit for bit
    # appending in two chunks (first_entry = entries already present) equals
    # one call, bit for bit
    z2 = rng.standard_normal((B, nb * m, d)).astype(np.float32)
    xd, zd = to_dev(x), to_dev(z2)
    whole = to_dev(_store(np.zeros((B, nb, d)), storage))
    parts = to_dev(_store(np.zeros((B, nb, d)), storage))
    csa.csa_compress(xd, zd, whole, m, 0)
    cut = 23 * m
    csa.csa_compress(xd[:, :cut], zd[:, :cut], parts, m, 0)
    csa.csa_compress(xd[:, cut:], zd[:, cut:], parts, m, cut // m)
    assert np.array_equal(from_dev(whole), from_dev(parts))


# ------------------------------------------------------------------- indexer

@pytest.mark.parametrize("kind,H_I,d_I", [("f32", 4, 64), ("f32", 64, 128), ("bf16", 64, 128),
                                         ("bf16", 20, 64), ("fp8", 64, 128), ("fp8", 7, 128),
                                         ("mxfp4", 64, 128), ("mxfp4", 7, 128)])
@pytest.mark.parametrize("act", ["relu", "identity"])
def test_indexer_parity(kind, H_I, d_I, act):
    say("indexer", kind, H_I, d_I, act)
    rng = np.random.default_rng(400 + H_I + d_I)
    B, T, m, n_cap = 2, 3, 4, 5000
    pos0 = np.array([4 * n_cap - 3, 37], np.int64)   # full cache / a short prefix
    storage = "f32" if kind == "f32" else "bf16"
    qi = _store(rng.standard_normal((B, T, H_I, d_I)), storage)
    ki = _store(rng.standard_normal((B, n_cap, d_I)), storage)
    w = rng.random((B, T, H_I)).astype(np.float32)
    qi_d, ki_d = to_dev(qi), to_dev(ki)
    qs = ks = None
    qv, kv = decode(qi), decode(ki)
    if kind == "fp8":
        qi_d, qs = csa.csa_quantize_fp8_rows(qi_d)
        ki_d, ks = csa.csa_quantize_fp8_rows(ki_d)
        qc, qsc = oracle.quantize_fp8_rows(qv.astype(np.float32))
        kcode, ksc = oracle.quantize_fp8_rows(kv.astype(np.float32))
        assert np.array_equal(from_dev(qi_d), qc) and np.array_equal(from_dev(ki_d), kcode)
        qv = oracle.e4m3_decode(qc) * qsc[..., None]
        kv = oracle.e4m3_decode(kcode) * ksc[..., None]
    if kind == "mxfp4":
        qi_d, qs = csa.csa_quantize_mxfp4_rows(qi_d)
        ki_d, ks = csa.csa_quantize_mxfp4_rows(ki_d)
        qc = oracle.quantize_mxfp4_rows(qv.astype(np.float32))
        kq = oracle.quantize_mxfp4_rows(kv.astype(np.float32))
        assert np.array_equal(from_dev(qi_d), qc[0]) and np.array_equal(from_dev(qs), qc[1])
        assert np.array_equal(from_dev(ki_d), kq[0]) and np.array_equal(from_dev(ks), kq[1])
        qv, kv = oracle.mxfp4_decode_rows(*qc), oracle.mxfp4_decode_rows(*kq)
    scores = torch.full((B, T, n_cap), float("nan"), device=DEV)
    csa.csa_index_scores(qi_d, to_dev(w), ki_d, to_dev(pos0), m, act, qi_scale=qs, ki_scale=ks,
                         scores=scores)
    got = from_dev(scores)
    worst = 0.0
    for b in range(B):
        pos = pos0[b] + np.arange(T)
        ref = oracle.indexer_scores(qv[b], w[b], kv[b], pos, m, act)
        V = oracle.visible_count(pos, m)
        for i in range(T):
            worst = max(worst, score_close(got[b, i, :V[i]], ref[i, :V[i]]))
            assert np.all(np.isnan(got[b, i, V[i]:])), "wrote past the visible entries"
    assert worst <= 1.0, worst


@pytest.mark.parametrize("m,d,H_I", [(4, 128, 64), (4, 64, 20), (1, 128, 64), (3, 256, 33)])
def test_decode_index_topk_fused_compress(m, d, H_I):
    """csa_decode_index_topk: the block completed by the query token is
    compressed inside the indexer launch (bit-identical to csa_compress on
    the same raw rows), then scored with the older entries; scores and
    indices equal csa_index_topk's on the updated cache, bit for bit, and
    the oracle's.  Sequences: a block completing at the full cache (entry
    in the last workgroup), at a short prefix (first workgroup), a token
    that completes no block, and a block whose first raw row lies before
    the raw buffer (left unwritten)."""
    say("decode index+topk fused compress", m, d, H_I)
    rng = np.random.default_rng(900 + m + d + H_I)
    B, n_cap, R, k = 4, 3000, 16, 64
    t = np.array([m * n_cap - 1, m * 37 - 1, m * 500 + (1 if m > 1 else 0), m * 900 - 1], np.int64)
    if m == 1:
        t[2] = 499  # every token completes a block when m == 1: a short prefix instead
    raw_pos0 = t - R + 1
    raw_pos0[3] = t[3] - m + 2                       # block starts one row before the buffer
    V = oracle.visible_count(t, m)
    kc0 = rng.standard_normal((B, n_cap, d))
    vc0 = rng.standard_normal((B, n_cap, d))
    for b in range(B):                               # sentinel where a block may land
        kc0[b, V[b] - 1] = 7.0
        vc0[b, V[b] - 1] = -7.0
    kc0, vc0 = bf16_codes(kc0), bf16_codes(vc0)
    kr = bf16_codes(rng.standard_normal((B, R, d)))
    vr = bf16_codes(rng.standard_normal((B, R, d)))
    zk = (rng.standard_normal((B, R, d)) * 2).astype(np.float32)
    zv = (rng.standard_normal((B, R, d)) * 2).astype(np.float32)
    qi = bf16_codes(rng.standard_normal((B, 1, H_I, d)))
    w = rng.random((B, 1, H_I)).astype(np.float32)
    kc, vc = to_dev(kc0), to_dev(vc0)
    pos0_d, raw_d = to_dev(t), to_dev(raw_pos0)
    sc, idx = csa.csa_decode_index_topk(to_dev(qi), to_dev(w), kc, vc, to_dev(kr), to_dev(vr),
                                        to_dev(zk), to_dev(zv), raw_d, pos0_d, m, k)
    torch.cuda.synchronize()
    kc1, vc1 = from_dev(kc), from_dev(vc)
    completes = [True, True, m == 1, False]
    for b in range(B):
        j = V[b] - 1
        rest = np.ones(n_cap, bool)
        rest[j] = False
        assert np.array_equal(kc1[b, rest], kc0[b, rest]) and np.array_equal(vc1[b, rest], vc0[b, rest])
        if not completes[b]:
            assert np.array_equal(kc1[b, j], kc0[b, j]) and np.array_equal(vc1[b, j], vc0[b, j]), b
            continue
        r0 = t[b] - m + 1 - raw_pos0[b]
        for name, x, z, got in (("k", kr, zk, kc1), ("v", vr, zv, vc1)):
            # csa_compress on the same rows: the same bits
            one = to_dev(bf16_codes(np.zeros((1, 1, d))))
            csa.csa_compress(to_dev(x[b:b + 1, r0:r0 + m].copy()), to_dev(z[b:b + 1, r0:r0 + m].copy()),
                             one, m, 0)
            assert np.array_equal(got[b, j], from_dev(one)[0, 0]), (name, b)
            xv = decode(x[b, r0:r0 + m])
            ref = oracle.compress(xv, z[b, r0:r0 + m], m)[0]
            assert np.all(np.abs(decode(got[b, j]) - ref) <= compress_bound(ref, xv[None], m)[0])
    # scores and indices: those of csa_index_topk on the updated cache
    sc2, idx2 = csa.csa_index_topk(to_dev(qi), to_dev(w), kc, pos0_d, m, k)
    got_s, got_i = from_dev(sc), from_dev(idx)
    ref_s2 = from_dev(sc2)
    for b in range(B):
        assert np.array_equal(got_s[b, 0, :V[b]], ref_s2[b, 0, :V[b]]), b
    assert np.array_equal(got_i, from_dev(idx2))
    kv = decode(kc1)
    for b in range(B):
        ref = oracle.indexer_scores(decode(qi[b]), w[b], kv[b], t[b:b + 1], m)
        assert score_close(got_s[b, 0, :V[b]], ref[0, :V[b]]) <= 1.0
        want = oracle.topk_select(got_s[b, 0, :V[b]].astype(np.float64), int(V[b]), k)
        assert np.array_equal(got_i[b, 0], want), b


def test_decode_index_topk_validation():
    say("decode index+topk validation")
    B, n_cap, R, d, m = 2, 256, 8, 128, 4
    z = lambda *s: torch.zeros(s, device=DEV)
    bf = lambda *s: torch.zeros(s, device=DEV, dtype=torch.bfloat16)
    pos = torch.full((B,), 100, dtype=torch.int64, device=DEV)
    args = dict(qi=bf(B, 1, 64, d), w=z(B, 1, 64), kc=bf(B, n_cap, d), vc=bf(B, n_cap, d),
                kr=bf(B, R, d), vr=bf(B, R, d), zk=z(B, R, d), zv=z(B, R, d), raw_pos0=pos,
                pos0=pos)
    with pytest.raises(ValueError):   # two query tokens
        csa.csa_decode_index_topk(**{**args, "qi": bf(B, 2, 64, d), "w": z(B, 2, 64)}, m=m, k=16)
    with pytest.raises(ValueError):   # logits of the wrong shape
        csa.csa_decode_index_topk(**{**args, "zk": z(B, R - 1, d)}, m=m, k=16)
    with pytest.raises(csa.CSAError):  # raw buffer shorter than a block
        csa.csa_decode_index_topk(**{**args, "kr": bf(B, 2, d), "vr": bf(B, 2, d),
                                     "zk": z(B, 2, d), "zv": z(B, 2, d)}, m=m, k=16)
    with pytest.raises(csa.CSAError):  # blocks longer than the fused path takes
        csa.csa_decode_index_topk(**args, m=8, k=16)


# --------------------------------------------------------------------- top-k

def _topk_case(scores, V, k):
    """Run csa_topk with m = 1 so that V(t) = t + 1 is set through pos0."""
    B, T, n_cap = scores.shape
    pos0 = (V[:, 0] - 1).astype(np.int64)
    assert np.all(V == (pos0[:, None] + np.arange(T) + 1))
    idx = csa.csa_topk(to_dev(scores.astype(np.float32)), to_dev(pos0), 1, k)
    got = from_dev(idx)
    for b in range(B):
        for i in range(T):
            want = oracle.topk_select(scores[b, i].astype(np.float64), int(min(V[b, i], n_cap)), k)
            assert np.array_equal(got[b, i], want), (b, i)
    return got


@pytest.mark.parametrize("path", ["split", "few_rows", "row", "row_long", "row_longer",
                                  "row_sorted"])
def test_topk_random_and_ties(path):
    """split: few rows longer than one workgroup handles (classify + finish
    kernels); few_rows: few short rows, one workgroup each; row: many rows
    (short ones, held in registers); row_long, row_longer: many rows read
    in batches of 32768 entries (two and three batches, the last ragged);
    row_sorted: many rows longer than the row kernel's output bitmap, whose
    selection is put in order by the sorting network instead."""
    say("topk", path)
    rng = np.random.default_rng(500)
    k = 100
    if path == "split":
        B, T, n_cap = 2, 4, 70000
    elif path == "few_rows":
        B, T, n_cap = 5, 4, 9000
    elif path == "row":
        B, T, n_cap = 1, 300, 3000
    elif path == "row_long":
        B, T, n_cap = 1, 264, 40000
    elif path == "row_longer":
        B, T, n_cap = 1, 260, 72000
    else:
        B, T, n_cap = 1, 258, 140000
    s = rng.standard_normal((B, T, n_cap)).astype(np.float32) * 30 + 140
    s[:, 1] = rng.integers(0, 40, size=s[:, 1].shape)          # heavy ties
    s[:, 2] = np.where(rng.random(s[:, 2].shape) < 0.5, -0.0, 0.0)  # signed zeros
    s[:, 2, ::7] = rng.standard_normal(s[:, 2, ::7].shape)
    V = np.zeros((B, T), np.int64)
    for b in range(B):
        start = n_cap - T - 3 * b if path != "row" else 40
        V[b] = start + np.arange(T)
    _topk_case(s, np.minimum(V, n_cap), k)


def test_topk_edge_rows():
    say("topk edges")
    rng = np.random.default_rng(501)
    # V <= k (all kept, -1 padding), V = k + 1, k = 1, and a row of equal
    # scores longer than the LDS candidate buffer (global fallback)
    cases = [(1, 64, 50), (1, 64, 64), (1, 64, 65), (1, 1, 3000), (2, 1024, 1025)]
    for B, k, v in cases:
        s = rng.standard_normal((B, 1, v + 5)).astype(np.float32)
        _topk_case(s, np.full((B, 1), v, np.int64), k)
    s = np.zeros((2, 1, 20000), np.float32)
    got = _topk_case(s, np.full((2, 1), 20000, np.int64), 1024)
    assert np.array_equal(got[0, 0], np.arange(1024))
    # equal scores on rows longer than one workgroup handles: the candidate
    # lists overflow and the finish kernel re-reads the row
    s = np.zeros((2, 1, 70000), np.float32)
    s[1, 0, 12345] = -1.0
    got = _topk_case(s, np.full((2, 1), 70000, np.int64), 2048)
    assert np.array_equal(got[0, 0], np.arange(2048))
    s = np.zeros((1, 300, 20000), np.float32)
    s[0, :, 5000] = 1.0
    got = _topk_case(s, np.arange(19700, 20000)[None], 16)
    assert np.array_equal(got[0, 0], np.r_[np.arange(15), 5000])


@pytest.mark.parametrize("n_cap,T", [(70000, 2), (9000, 3), (3000, 300), (40000, 264)])
def test_topk_cut_inside_small_tie_group(n_cap, T):
    """The k-th largest score shared by a handful of entries (fewer than 64
    share its top 20 key bits, the case the cut search ranks in one wave):
    the lowest indices among them win, on every top-k path."""
    say("topk small tie group at the cut", n_cap, T)
    rng = np.random.default_rng(502 + T)
    k = 100
    s = (rng.standard_normal((1, T, n_cap)) * 30 + 140).astype(np.float32)
    for i in range(T):
        order = np.argsort(-s[0, i], kind="stable")
        group = order[k - 4:k + 6]                 # ranks 97 .. 106 -> one value
        s[0, i, group] = s[0, i, order[k - 1]]
    V = n_cap - T + 1 + np.arange(T, dtype=np.int64)[None]   # the last row sees all
    _topk_case(s, V, k)


def test_topk_split_lists_past_prefetch():
    """Split path: the finishing kernel prefetches a prefix of every slice's
    list; here one slice holds almost all the selected entries, so its list
    is fetched mostly in the second step."""
    say("topk concentrated slice")
    rng = np.random.default_rng(503)
    s = (rng.standard_normal((2, 1, 70000)) * 30 + 140).astype(np.float32)
    s[0, 0, 4096:8192] += 400.0            # slice 1 holds the top 4096
    s[1, 0, 60000:60000 + 3000] = 1000.0   # 3000 equal maxima in slices 14-15
    _topk_case(s, np.full((2, 1), 70000, np.int64), 2048)


def test_topk_long_rows_decode_shape():
    say("topk long rows")
    rng = np.random.default_rng(502)
    s = (rng.standard_normal((4, 1, 262144)) * 31 + 141).astype(np.float32)
    _topk_case(s, np.full((4, 1), 262144, np.int64), 1024)


# ----------------------------------------------------------------- attention

def _attend_case(storage, B, T, H, d, N, k, W, R, raw_off, seed, hca_m=0, fill=0.8):
    rng = np.random.default_rng(seed)
    kc = _store(rng.standard_normal((B, N, d)), storage)
    vc = _store(rng.standard_normal((B, N, d)), storage)
    kr = _store(rng.standard_normal((B, R, d)), storage)
    vr = _store(rng.standard_normal((B, R, d)), storage)
    q = _store(rng.standard_normal((B, T, H, d)), storage)
    m = hca_m if hca_m else 4
    pos0 = np.array([raw_off[b] + R - T for b in range(B)], np.int64)
    raw_pos0 = np.array(raw_off, np.int64)
    scale = 1.0 / math.sqrt(d)
    idx = None
    if not hca_m:
        idx = np.full((B, T, k), -1, np.int32)
        for b in range(B):
            for i in range(T):
                V = int(min(N, (pos0[b] + i + 1) // m))
                n = min(V, int(rng.integers(int(fill * k), k + 1)))
                idx[b, i, :n] = np.sort(rng.choice(V, size=n, replace=False))
    args = (to_dev(q), to_dev(kc), to_dev(vc))
    if hca_m:
        out, lse = csa.hca_attend(*args, hca_m, to_dev(kr), to_dev(vr), to_dev(raw_pos0),
                                  to_dev(pos0), W, scale)
    else:
        out, lse = csa.csa_attend(*args, to_dev(idx), to_dev(kr), to_dev(vr), to_dev(raw_pos0),
                                  to_dev(pos0), W, scale)
    out, lse = from_dev(out), from_dev(lse)
    errs, rels = [], []
    for b in range(B):
        pos = pos0[b] + np.arange(T)
        if hca_m:
            ref, ref_lse = oracle.hca_attend(decode(q[b]), decode(kc[b]), decode(vc[b]),
                                             decode(kr[b]), decode(vr[b]), raw_pos0[b], pos,
                                             hca_m, W, scale)
        else:
            ref, ref_lse = oracle.attend(decode(q[b]), decode(kc[b]), decode(vc[b]), idx[b],
                                         decode(kr[b]), decode(vr[b]), raw_pos0[b], pos, W, scale)
        errs.append(np.max(np.abs(out[b] - ref)))
        errs.append(np.max(np.abs(lse[b] - ref_lse)))
        rels.append(rel_l2(out[b], ref))
    return max(errs), max(rels)


@pytest.mark.parametrize("storage,H,d", [("f32", 8, 64), ("f32", 64, 128), ("bf16", 64, 128),
                                         ("bf16", 16, 64), ("bf16", 40, 128)])
@pytest.mark.parametrize("rows", ["few", "many", "wide"])
def test_attend_parity(storage, H, d, rows):
    """few: split rows and the merge; many: one workgroup per query; wide:
    a grid of 600 rows, which bf16 at d 128 runs two workgroups per CU."""
    say("attend", storage, H, d, rows)
    if rows == "few":   # split over several workgroups + merge
        B, T, k, N, W, R = 3, 2, 700, 3000, 128, 200
    elif rows == "many":  # one workgroup per query
        B, T, k, N, W, R = 1, 300, 64, 600, 32, 400
    else:
        B, T, k, N, W, R = 1, 600, 96, 1200, 48, 800
    err, rel = _attend_case(storage, B, T, H, d, N, k, W, R, [100 * b + 2500 for b in range(B)]
                            if rows == "few" else [2000], seed=600 + H + d)
    tol = 1e-4 if storage == "f32" else 2e-2
    assert err <= tol, err
    assert rel <= (1e-5 if storage == "f32" else 1e-2), rel


@pytest.mark.parametrize("storage", ["f32", "bf16"])
def test_attend_window_edges(storage):
    """Queries near position 0 (window shorter than W, nothing compressed
    yet) and an empty selection."""
    say("attend edges", storage)
    err, _ = _attend_case(storage, 1, 9, 16, 64, 8, 4, 5, 9, [0], seed=700, fill=0.0)
    assert err <= (1e-4 if storage == "f32" else 2e-2)
    # t = 0: the only key is raw token 0, so O = v_0 exactly
    rng = np.random.default_rng(701)
    d, H = 64, 16
    q = _store(rng.standard_normal((1, 1, H, d)), storage)
    v = _store(rng.standard_normal((1, 1, d)), storage)
    kk = _store(rng.standard_normal((1, 1, d)), storage)
    kc = to_dev(_store(np.zeros((1, 4, d)), storage))
    zero = to_dev(np.zeros(1, np.int64))
    out, lse = csa.csa_attend(to_dev(q), kc, kc, to_dev(np.full((1, 1, 4), -1, np.int32)),
                              to_dev(kk), to_dev(v), zero, zero, 32, 0.125)
    assert np.array_equal(from_dev(out)[0, 0], np.tile(decode(v)[0, 0], (H, 1)).astype(np.float32))


@pytest.mark.parametrize("storage", ["f32", "bf16"])
def test_attend_window_only(storage):
    """Sliding-window-only attention (the hybrid stack's first layers):
    k = 0, no compressed entry is read."""
    say("attend window only", storage)
    err, rel = _attend_case(storage, 2, 3, 64, 128, 1, 0, 128, 300, [1000, 5000], seed=720)
    assert err <= (1e-4 if storage == "f32" else 2e-2), err
    assert rel <= (1e-5 if storage == "f32" else 1e-2), rel


@pytest.mark.parametrize("storage,m", [("bf16", 128), ("bf16", 4), ("f32", 4)])
def test_hca_parity(storage, m):
    say("hca", storage, m)
    B, T, H, d, N, W, R = 2, 2, 64, 128, 1500, 128, 300
    raw = [N * m - 5 - R + T, 40 * m]
    err, rel = _attend_case(storage, B, T, H, d, N, 0, W, R, raw, seed=800 + m, hca_m=m)
    assert err <= (1e-4 if storage == "f32" else 2e-2), err
    assert rel <= (1e-5 if storage == "f32" else 1e-2), rel


def test_workspaces_are_reusable_across_calls():
    """Every call leaves a workspace ready for the next: reusing one
    workspace for several top-k / attention calls on different data gives
    the same results as fresh workspaces, and the parts read before being
    written (histograms, counters) are zero afterwards."""
    say("workspace reuse")
    rng = np.random.default_rng(900)
    B, T, n_cap, k = 3, 2, 9000, 256
    ws = csa.workspace(csa.csa_topk_workspace_size(B, T, n_cap, k), DEV)
    pos0 = to_dev(np.array([n_cap - 2, 5000, 3000], np.int64))
    for trial in range(3):
        s = (rng.standard_normal((B, T, n_cap)) * (trial + 1)).astype(np.float32)
        if trial == 1:
            s[0] = 0.0  # candidate overflow path on one sequence
        got = csa.csa_topk(to_dev(s), pos0, 1, k, ws=ws)
        ref = csa.csa_topk(to_dev(s), pos0, 1, k)
        assert torch.equal(got, ref), trial
    # the histogram and counters (the part read before being written) are zero
    hist_bytes = B * T * (4096 + 4) * 4
    assert int(ws[:hist_bytes].count_nonzero().item()) == 0
    # fused indexer histogram + top-k with a reused workspace
    H_I, d_I = 64, 128
    qi = to_dev(bf16_codes(rng.standard_normal((B, T, H_I, d_I))))
    ki = to_dev(bf16_codes(rng.standard_normal((B, n_cap, d_I))))
    w = to_dev(rng.random((B, T, H_I)).astype(np.float32))
    pos4 = to_dev(np.array([4 * n_cap - 5, 4 * 5000, 4 * 3000], np.int64))
    for trial in range(3):
        sc = csa.csa_index_scores(qi, w, ki, pos4, 4, topk_ws=ws, k=k)
        fused = csa.csa_topk(sc, pos4, 4, k, ws=ws, hist_ready=True)
        plain = csa.csa_topk(sc, pos4, 4, k)
        assert torch.equal(fused, plain), trial
    torch.cuda.synchronize()
    assert int(ws[:hist_bytes].count_nonzero().item()) == 0
    # attention with split partials and a reused workspace
    H, d, W, R = 64, 128, 128, 200
    Bq, Tq, N, ka = 2, 1, 3000, 700
    aws = csa.workspace(csa.csa_attend_workspace_size(Bq, Tq, H, d, ka, W), DEV)
    for trial in range(3):
        q = to_dev(bf16_codes(rng.standard_normal((Bq, Tq, H, d))))
        kc = to_dev(bf16_codes(rng.standard_normal((Bq, N, d))))
        vc = to_dev(bf16_codes(rng.standard_normal((Bq, N, d))))
        kr = to_dev(bf16_codes(rng.standard_normal((Bq, R, d))))
        vr = to_dev(bf16_codes(rng.standard_normal((Bq, R, d))))
        idx = np.sort(rng.choice(N, size=(Bq, Tq, ka)), axis=-1).astype(np.int32)
        raw = to_dev(np.array([5000, 5100], np.int64))
        p0 = to_dev(np.array([5000 + R - 1, 5100 + R - 1], np.int64))
        a, al = csa.csa_attend(q, kc, vc, to_dev(idx), kr, vr, raw, p0, W, 0.088, ws=aws)
        b_, bl = csa.csa_attend(q, kc, vc, to_dev(idx), kr, vr, raw, p0, W, 0.088)
        assert torch.equal(a, b_) and torch.equal(al, bl), trial


@pytest.mark.parametrize("kind,H_I", [("bf16", 64), ("bf16", 40), ("fp8", 64), ("mxfp4", 64)])
@pytest.mark.parametrize("act", ["relu", "identity"])
def test_indexer_prefill_parity(kind, H_I, act):
    """Many query tokens per sequence (the multi-token MFMA tile path): a
    ragged token count, visibility growing across the chunk and, for one
    sequence, entries cut by the cache capacity."""
    say("indexer prefill", kind, H_I, act)
    rng = np.random.default_rng(1000 + H_I)
    B, T, m, n_cap, d_I = 2, 21, 4, 3000, 128
    pos0 = np.array([4 * 2990, 4 * 1000 - 7], np.int64)
    qi = bf16_codes(rng.standard_normal((B, T, H_I, d_I)))
    ki = bf16_codes(rng.standard_normal((B, n_cap, d_I)))
    w = rng.random((B, T, H_I)).astype(np.float32)
    qi_d, ki_d = to_dev(qi), to_dev(ki)
    qs = ks = None
    qv, kv = decode(qi), decode(ki)
    if kind == "fp8":
        qi_d, qs = csa.csa_quantize_fp8_rows(qi_d)
        ki_d, ks = csa.csa_quantize_fp8_rows(ki_d)
        qv = oracle.e4m3_decode(from_dev(qi_d)) * from_dev(qs)[..., None]
        kv = oracle.e4m3_decode(from_dev(ki_d)) * from_dev(ks)[..., None]
    if kind == "mxfp4":   # (many tokens take the decode kernel for MXFP4)
        qi_d, qs = csa.csa_quantize_mxfp4_rows(qi_d)
        ki_d, ks = csa.csa_quantize_mxfp4_rows(ki_d)
        qv = oracle.mxfp4_decode_rows(from_dev(qi_d), from_dev(qs))
        kv = oracle.mxfp4_decode_rows(from_dev(ki_d), from_dev(ks))
    scores = torch.full((B, T, n_cap), float("nan"), device=DEV)
    csa.csa_index_scores(qi_d, to_dev(w), ki_d, to_dev(pos0), m, act, qi_scale=qs, ki_scale=ks,
                         scores=scores)
    got = from_dev(scores)
    worst = 0.0
    for b in range(B):
        pos = pos0[b] + np.arange(T)
        V = np.minimum(oracle.visible_count(pos, m), n_cap)
        ref = oracle.indexer_scores(qv[b], w[b], kv[b][:n_cap], np.minimum(pos, 4 * n_cap - 1), m,
                                    act)
        for i in range(T):
            worst = max(worst, score_close(got[b, i, :V[i]], ref[i, :V[i]]))
            assert np.all(np.isnan(got[b, i, V[i]:])), "wrote past the visible entries"
    assert worst <= 1.0, worst
