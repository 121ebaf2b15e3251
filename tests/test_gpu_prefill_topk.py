"""The many-row top-k fed by the prefill indexer's coarse histograms
(csa_index_scores given a top-k workspace for more than 256 query rows,
then csa_topk with hist_ready): every row's selection must equal the
oracle's top-k of the GPU's own scores bit for bit.  The cases cover rows
held in registers (n_cap <= 32768) and rows read in batches (two and
three of them), k-th keys in
the upper and in the lower half of their coarse bucket (both asserted to
occur), ties that overflow the LDS candidate list (the exact
re-classification), fp8 keys, the per-row flags (set by the indexer,
cleared by the top-k) and a flag left by an indexer call that another
path overrides."""

import numpy as np
import pytest
import torch

from conftest import ensure_library
from gpu_util import DEV, bf16_codes, from_dev, say, to_dev

import oracle

pytestmark = pytest.mark.gpu

ensure_library()
import long_context_sparse_16_amd as csa  # noqa: E402

COARSE_BINS = 2048


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _keys(x):
    """Order-preserving uint32 keys of float32 scores (+-0 equal)."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    k = np.where(u >> 31 == 1, (~u) & 0xffffffff, u | 0x80000000)
    k = np.where((u << 1) & 0xffffffff == 0, 0x80000000, k)
    return k.astype(np.uint64)


def _flags(tws, rows):
    return tws[rows * COARSE_BINS * 4:(rows * COARSE_BINS + rows) * 4].view(torch.int32)


def _inputs(seed, B, T, n_cap, H_I=16, key_rows=None, fp8=False):
    rng = np.random.default_rng(seed)
    qi = to_dev(bf16_codes(rng.standard_normal((B, T, H_I, 128))))
    if key_rows is None:
        ki = rng.standard_normal((B, n_cap, 128))
    else:
        ki = key_rows[rng.integers(0, len(key_rows), size=(B, n_cap))]
    ki = to_dev(bf16_codes(ki))
    w = to_dev(rng.random((B, T, H_I)).astype(np.float32))
    qs = ks = None
    if fp8:
        qi, qs = csa.csa_quantize_fp8_rows(qi)
        ki, ks = csa.csa_quantize_fp8_rows(ki)
    return qi, w, ki, qs, ks


def _check_rows(scores, idx, pos0, T, m, k):
    """Every row against the oracle; returns which half of the coarse
    bucket held each row's k-th key (for rows with V > k)."""
    s = from_dev(scores)
    ix = from_dev(idx)
    halves = set()
    for b in range(s.shape[0]):
        for i in range(T):
            V = int(min(s.shape[2], oracle.visible_count(np.array([pos0[b] + i]), m)[0]))
            want = oracle.topk_select(s[b, i].astype(np.float64), V, k)
            assert np.array_equal(ix[b, i], want), (b, i)
            if V > k:
                kth = np.sort(_keys(s[b, i, :V]))[::-1][k - 1]
                halves.add(int((kth >> 20) & 1))
    return halves


CASES = {
    # name: (B, T, n_cap, pos0, k, extra)
    "regs_rows": (2, 160, 6000, [4 * 5000, 4 * 6000 - 200], 512, {}),
    "long_rows": (1, 264, 40000, [4 * 39000], 1024, {}),
    "fp8_long": (1, 272, 36000, [4 * 35500], 1024, {"fp8": True}),
    "batched_rows": (1, 264, 72000, [4 * 71000], 1024, {}),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_prefill_topk_from_coarse_histograms(name):
    B, T, n_cap, pos0, k, extra = CASES[name]
    say("prefill top-k, coarse histograms", name)
    qi, w, ki, qs, ks = _inputs(sum(map(ord, name)), B, T, n_cap, **extra)
    p0 = torch.tensor(pos0, dtype=torch.int64, device=DEV)
    rows = B * T
    tws = csa.workspace(csa.csa_topk_workspace_size(B, T, n_cap, k), DEV)
    assert tws.numel() >= rows * (COARSE_BINS + 1) * 4
    for call in range(2):
        scores = csa.csa_index_scores(qi, w, ki, p0, 4, qi_scale=qs, ki_scale=ks, topk_ws=tws,
                                      k=k)
        torch.cuda.synchronize()
        assert int(_flags(tws, rows).sum()) == rows, "the indexer writes every row's histogram"
        idx = csa.csa_topk(scores, p0, 4, k, ws=tws, hist_ready=True)
        torch.cuda.synchronize()
        assert int(_flags(tws, rows).abs().sum()) == 0, "the top-k clears every flag"
        halves = _check_rows(scores, idx, pos0, T, 4, k)
    assert halves == {0, 1}, f"both halves of the coarse bucket should occur, saw {halves}"


@pytest.mark.parametrize("n_cap,T", [(20000, 264), (40000, 260), (72000, 260)])
def test_prefill_topk_coarse_candidates_overflow(n_cap, T):
    """Keys from 2 distinct rows: every score takes one of two values per
    query, so the coarse bucket holds far more candidates than the LDS
    list; the row is classified again against the exact bucket."""
    say("prefill top-k, coarse overflow", n_cap, T)
    rng = np.random.default_rng(n_cap)
    key_rows = rng.standard_normal((2, 128))
    B, k = 1, 1024
    pos0 = [4 * n_cap - 1 - T]
    qi, w, ki, qs, ks = _inputs(7 + n_cap, B, T, n_cap, key_rows=key_rows)
    p0 = torch.tensor(pos0, dtype=torch.int64, device=DEV)
    tws = csa.workspace(csa.csa_topk_workspace_size(B, T, n_cap, k), DEV)
    scores = csa.csa_index_scores(qi, w, ki, p0, 4, topk_ws=tws, k=k)
    idx = csa.csa_topk(scores, p0, 4, k, ws=tws, hist_ready=True)
    torch.cuda.synchronize()
    _check_rows(scores, idx, pos0, T, 4, k)


def test_prefill_topk_flags_overridden_by_other_path():
    """A bf16 indexer call leaves its histograms and flags in the workspace;
    an fp32 indexer call of the same sizes (which the prefill kernel does
    not take) must clear the flags, so the top-k that follows reads its own
    rows instead of the stale histograms."""
    say("prefill top-k, stale flags")
    B, T, n_cap, k = 1, 272, 9000, 512
    pos0 = [4 * 8900]
    qi, w, ki, _, _ = _inputs(31, B, T, n_cap)
    p0 = torch.tensor(pos0, dtype=torch.int64, device=DEV)
    tws = csa.workspace(csa.csa_topk_workspace_size(B, T, n_cap, k), DEV)
    csa.csa_index_scores(qi, w, ki, p0, 4, topk_ws=tws, k=k)
    torch.cuda.synchronize()
    assert int(_flags(tws, B * T).sum()) == B * T
    rng = np.random.default_rng(32)
    qf = to_dev(rng.standard_normal((B, T, 16, 128)).astype(np.float32))
    kf = to_dev(rng.standard_normal((B, n_cap, 128)).astype(np.float32))
    scores = csa.csa_index_scores(qf, w, kf, p0, 4, topk_ws=tws, k=k)
    torch.cuda.synchronize()
    assert int(_flags(tws, B * T).abs().sum()) == 0
    idx = csa.csa_topk(scores, p0, 4, k, ws=tws, hist_ready=True)
    torch.cuda.synchronize()
    _check_rows(scores, idx, pos0, T, 4, k)
