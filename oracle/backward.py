"""Plain fp64 gradients of the compressor and of core attention (the
backward pass of the hot path).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages describe a model trained end to end: the compressor is learned
(octagono.org "Hybrid Attention: CSA and HCA": a learned token-level
compressor; "DeepSeek V4 technical review", takeshell.com, section 2.1:
weighted aggregation of every m tokens) and the indexer's QK path is
trained quantization-aware (dataforcee.us "Muon Optimizer and FP4 QAT";
takeshell.com section 5).  They give no formula for the backward pass, so
these functions are the derivatives of this package's forward definitions
(``compress`` and ``attend``), written out by the chain rule:

attention, one query row t and head h over its key list (keys K, values V,
logits s = scale * K q, probabilities p = softmax(s), output o = p V):
    dp   = V dout            (one value per key)
    D    = dout . o
    ds   = p * (dp - D)
    dq   = scale * ds K
    dK  += scale * ds (outer) q      (per key row; summed over heads/rows)
    dV  += p (outer) dout
compressor, one block and channel (w = softmax of the m logits z,
c = sum_i w_i x_i):
    dx_i = w_i dc
    dz_i = w_i (x_i - c) dc

No gradient flows through the top-k selection (a discrete choice); the
selected index lists are an input, as in the forward.  Gradients of keys and
values that several query rows select are summed.
"""

from __future__ import annotations

import numpy as np

from .csa import hca_indices


def attend_backward(q, kc, vc, idx, kr, vr, raw_pos0: int, pos, W: int, scale: float, dout):
    """Gradients of ``attend``'s output with respect to its inputs.

    Arguments as ``attend`` plus dout [T, H, d], the gradient of the loss
    with respect to the output O.  Returns a dict with dq [T, H, d],
    dkc, dvc [N, d] and dkr, dvr [R, d] (rows never attended get zeros).
    """
    q = np.asarray(q, dtype=np.float64)
    kc = np.asarray(kc, dtype=np.float64)
    vc = np.asarray(vc, dtype=np.float64)
    kr = np.asarray(kr, dtype=np.float64)
    vr = np.asarray(vr, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    idx = np.asarray(idx)
    pos = np.asarray(pos, dtype=np.int64)
    T, H, d = q.shape
    R = kr.shape[0]
    dq = np.zeros_like(q)
    dkc, dvc = np.zeros_like(kc), np.zeros_like(vc)
    dkr, dvr = np.zeros_like(kr), np.zeros_like(vr)
    for t in range(T):
        sel = idx[t][idx[t] >= 0].astype(np.int64)
        rows = np.arange(max(0, pos[t] - W + 1), pos[t] + 1) - raw_pos0
        assert rows.size == 0 or (rows.min() >= 0 and rows.max() < R), "window outside raw buffer"
        keys = np.concatenate([kc[sel], kr[rows]], axis=0)
        vals = np.concatenate([vc[sel], vr[rows]], axis=0)
        s = (q[t] @ keys.T) * scale                      # [H, n]
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        o = p @ vals                                     # [H, d]
        dp = dout[t] @ vals.T                            # [H, n]
        D = (dout[t] * o).sum(axis=1, keepdims=True)     # [H, 1]
        ds = p * (dp - D)
        dq[t] = scale * (ds @ keys)
        dkeys = scale * (ds.T @ q[t])                    # [n, d]
        dvals = p.T @ dout[t]                            # [n, d]
        ns = sel.size
        np.add.at(dkc, sel, dkeys[:ns])
        np.add.at(dvc, sel, dvals[:ns])
        np.add.at(dkr, rows, dkeys[ns:])
        np.add.at(dvr, rows, dvals[ns:])
    return {"dq": dq, "dkc": dkc, "dvc": dvc, "dkr": dkr, "dvr": dvr}


def hca_attend_backward(q, kc, vc, kr, vr, raw_pos0: int, pos, m: int, W: int, scale: float,
                        dout):
    """Gradients of ``hca_attend`` (every visible entry selected)."""
    return attend_backward(q, kc, vc, hca_indices(pos, m), kr, vr, raw_pos0, pos, W, scale, dout)


def compress_backward(x, logits, m: int, dc):
    """Gradients of ``compress`` with respect to the tokens x [n, d] and the
    logits [n, d], for dc [n/m, d] the gradient with respect to the
    compressed rows.  Returns (dx, dlogits)."""
    x = np.asarray(x, dtype=np.float64)
    z = np.asarray(logits, dtype=np.float64)
    dc = np.asarray(dc, dtype=np.float64)
    n, d = x.shape
    assert n % m == 0 and dc.shape == (n // m, d)
    xb = x.reshape(n // m, m, d)
    zb = z.reshape(n // m, m, d)
    w = np.exp(zb - zb.max(axis=1, keepdims=True))
    w /= w.sum(axis=1, keepdims=True)
    c = (w * xb).sum(axis=1, keepdims=True)
    dx = w * dc[:, None, :]
    dz = w * (xb - c) * dc[:, None, :]
    return dx.reshape(n, d), dz.reshape(n, d)
