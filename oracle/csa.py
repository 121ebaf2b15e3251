"""Plain fp64 definition of Compressed Sparse Attention (CSA) and of its
heavily compressed dense variant (HCA).

TEST INFRASTRUCTURE ONLY (see the package docstring).

All arithmetic is float64 over the exact decoded values of the stored inputs
(bf16 / fp8 codes are decoded by ``oracle.codecs`` before they get here).
Every function works on one sequence; callers loop over the batch.

Method, as the pages state it (cited by page title and section):

1. Compression -- every m tokens of KV become one entry by a learned,
   token-level weighted aggregation, shrinking the sequence to 1/m of its
   length ("DeepSeek V4 technical review", takeshell.com, section 2.1;
   octagono.org "Hybrid Attention: CSA and HCA").
2. Lightning Indexer -- indexer queries per query token are scored against
   the compressed entries (takeshell.com 2.1; 64 heads x 128 dims for
   V4-Pro in the "Key parameters" list there).
3. Top-k -- the k highest-scoring compressed entries are kept (k = 1024 for
   V4-Pro; takeshell.com 2.1, octagono.org "Hybrid Attention").
4. Core attention over only the selected entries, together with a sliding
   window over the most recent raw tokens (128 on octagono.org; "both CSA
   and HCA include a sliding window attention branch", dataforcee.us
   "Hybrid Attention: CSA and HCA").
5. HCA -- compression with m' >> m (m' = 128, takeshell.com 2.2) followed by
   dense attention over all compressed entries, no selection
   (octagono.org "Hybrid Attention"; dataforcee.us "Hybrid Attention").

Readings taken where the pages are silent (each is listed with its reason in
the repository's design notes): softmax-over-the-block weights from caller
logits per (token, channel); block j is visible to query position t iff it
ends at or before t, i.e. V(t) = floor((t+1)/m); indexer score
S[t,j] = sum_h w[t,h] * relu(q_I[t,h] . k_I[j]) (identity also offered);
top-k ordered by (score desc, index asc), emitted ascending, padded with -1;
the window is the W raw positions ending at t, concatenated with the
selected entries into one softmax with no de-duplication; one KV head shared
by all query heads; scale given by the caller (1/sqrt(d) in every workload).
"""

from __future__ import annotations

import numpy as np

RELU = "relu"
IDENTITY = "identity"


def visible_count(t, m: int):
    """Number of compressed entries visible to query position t.

    Block j covers raw positions j*m .. j*m+m-1 and is visible iff its last
    position is <= t, so V(t) = floor((t + 1) / m).
    """
    return (np.asarray(t, dtype=np.int64) + 1) // int(m)


def compress(x, logits, m: int) -> np.ndarray:
    """Token-level compressor: each non-overlapping block of m rows of ``x``
    ([n, d], n a multiple of m) becomes one row.

    For block j and channel c the weights are the softmax over the m tokens
    of logits[j*m + i, c]; the entry is sum_i weight_i * x[j*m + i, c].
    """
    x = np.asarray(x, dtype=np.float64)
    z = np.asarray(logits, dtype=np.float64)
    n, d = x.shape
    assert z.shape == (n, d)
    assert n % m == 0, "only complete blocks are compressed"
    nb = n // m
    xb = x.reshape(nb, m, d)
    zb = z.reshape(nb, m, d)
    a = np.exp(zb - zb.max(axis=1, keepdims=True))
    weights = a / a.sum(axis=1, keepdims=True)
    return (weights * xb).sum(axis=1)


def indexer_scores(qi, w, ki, pos, m: int, act: str = RELU) -> np.ndarray:
    """Lightning Indexer scores for one sequence.

    qi: [T, H_I, d_I] indexer queries (dequantized), w: [T, H_I] head
    weights, ki: [N, d_I] indexer keys (dequantized), pos: [T] absolute
    query positions.  Returns S [T, N] with
    S[t, j] = sum_h w[t, h] * phi(qi[t, h] . ki[j])  for j < V(t),
    and NaN for entries that are not yet visible.  phi is ReLU or identity.
    """
    qi = np.asarray(qi, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    ki = np.asarray(ki, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    T, H, dI = qi.shape
    N = ki.shape[0]
    assert w.shape == (T, H) and ki.shape[1] == dI and pos.shape == (T,)
    V = visible_count(pos, m)
    assert np.all(V <= N), "query position beyond the compressed cache"
    S = np.full((T, N), np.nan)
    for t in range(T):
        dots = qi[t] @ ki[: V[t]].T  # [H, V]
        if act == RELU:
            dots = np.maximum(dots, 0.0)
        elif act != IDENTITY:
            raise ValueError(act)
        S[t, : V[t]] = w[t] @ dots
    return S


def topk_select(scores_row, n_visible: int, k: int) -> np.ndarray:
    """Per-query top-k over the first ``n_visible`` entries of one score row.

    The min(k, n_visible) entries with the largest score are kept, equal
    scores going to the lower entry index; they are returned in ascending
    index order and the row is padded to length k with -1.
    """
    s = np.asarray(scores_row, dtype=np.float64)[:n_visible]
    assert np.all(np.isfinite(s)), "scores must be finite"
    j = np.arange(n_visible)
    # +0.0 and -0.0 compare equal, so such ties also fall to the index.
    order = np.lexsort((j, -s))
    keep = np.sort(order[: min(k, n_visible)])
    out = np.full(k, -1, dtype=np.int32)
    out[: keep.size] = keep
    return out


def attend(q, kc, vc, idx, kr, vr, raw_pos0: int, pos, W: int, scale: float):
    """Core attention of one sequence over the selected compressed entries
    plus the sliding window, in one softmax.

    q: [T, H, d]; kc, vc: [N, d] compressed K/V; idx: [T, k] selected entry
    indices (-1 = unused); kr, vr: [R, d] raw K/V holding positions
    raw_pos0 .. raw_pos0+R-1; pos: [T] query positions; W: window length.
    For query t the key set is [kc[j] for j in idx[t] if j >= 0] followed by
    kr at positions max(0, t-W+1) .. t.  Every query head uses the same key
    set (one shared KV head).  Returns (O [T, H, d], lse [T, H]) where lse is
    the natural-log sum of exp(logits).
    """
    q = np.asarray(q, dtype=np.float64)
    kc = np.asarray(kc, dtype=np.float64)
    vc = np.asarray(vc, dtype=np.float64)
    kr = np.asarray(kr, dtype=np.float64)
    vr = np.asarray(vr, dtype=np.float64)
    idx = np.asarray(idx)
    pos = np.asarray(pos, dtype=np.int64)
    T, H, d = q.shape
    R = kr.shape[0]
    O = np.zeros((T, H, d))
    lse = np.zeros((T, H))
    for t in range(T):
        sel = idx[t][idx[t] >= 0].astype(np.int64)
        p = np.arange(max(0, pos[t] - W + 1), pos[t] + 1) - raw_pos0
        assert p.size == 0 or (p.min() >= 0 and p.max() < R), "window outside raw buffer"
        keys = np.concatenate([kc[sel], kr[p]], axis=0)
        vals = np.concatenate([vc[sel], vr[p]], axis=0)
        logits = (q[t] @ keys.T) * scale  # [H, n_keys]
        mx = logits.max(axis=1, keepdims=True)
        e = np.exp(logits - mx)
        den = e.sum(axis=1, keepdims=True)
        O[t] = (e @ vals) / den
        lse[t] = mx[:, 0] + np.log(den[:, 0])
    return O, lse


def hca_indices(pos, m: int) -> np.ndarray:
    """Index lists for HCA: every visible entry 0 .. V(t)-1, padded with -1
    to the longest list."""
    V = visible_count(np.asarray(pos, dtype=np.int64), m)
    width = max(int(V.max()), 1) if V.size else 1
    out = np.full((V.size, width), -1, dtype=np.int32)
    for t, v in enumerate(V):
        out[t, :v] = np.arange(v)
    return out


def hca_attend(q, kc, vc, kr, vr, raw_pos0: int, pos, m: int, W: int, scale: float):
    """HCA: dense attention over all visible compressed entries (compression
    ratio m') plus the sliding window."""
    return attend(q, kc, vc, hca_indices(pos, m), kr, vr, raw_pos0, pos, W, scale)


def csa_forward(k_raw, v_raw, logits, qi, w, q, m: int, k: int, W: int, scale: float,
                act: str = RELU):
    """CSA over one sequence prefilled from position 0: compress K and V
    with the shared logits (indexer keys are the compressed keys), score,
    select, attend.  Returns a dict of every intermediate."""
    n = np.asarray(k_raw).shape[0]
    pos = np.arange(n)
    kc = compress(k_raw, logits, m)
    vc = compress(v_raw, logits, m)
    S = indexer_scores(qi, w, kc, pos, m, act)
    V = visible_count(pos, m)
    idx = np.stack([topk_select(S[t], int(V[t]), k) for t in range(n)])
    O, lse = attend(q, kc, vc, idx, k_raw, v_raw, 0, pos, W, scale)
    return {"kc": kc, "vc": vc, "scores": S, "idx": idx, "out": O, "lse": lse}
