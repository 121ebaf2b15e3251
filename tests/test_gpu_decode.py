"""The whole decode step in one call (csa_decode), and the top-k selection
with attention (csa_select_attend), against the same step as separate calls
(csa_index_topk, then csa_attend): scores, indices, outputs and lse must be
bit-identical -- the selection made inside the attention launch is the
top-k kernels' exact one, and the attention arithmetic is shared.  The
cases cover rows that keep every visible entry, ragged positions per
sequence, long rows, ties that fill the top-k's candidate lists, fp32 /
bf16 / fp8 / MXFP4 indexer keys, the block compression of a
block-completing token, and repeated calls on one workspace (the top-k
histograms inside it must come back to zero).  The selection is also
checked against the oracle's top-k of the GPU's own scores."""

import numpy as np
import pytest
import torch

from conftest import ensure_library
from gpu_util import DEV, bf16_codes, say, to_dev

import oracle

pytestmark = pytest.mark.gpu

ensure_library()
import long_context_sparse_16_amd as csa  # noqa: E402


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _inputs(seed, B, T, n_cap, pos0, d=128, H=8, H_I=4, d_I=128, W=16, storage="bf16",
            ki_kind=None, key_values=None, m=4):
    """Random decode inputs; ki_kind None (= kc), "fp8" or "mxfp4";
    key_values: draw the compressed keys from this small set of rows (ties)."""
    rng = np.random.default_rng(seed)
    st = (lambda a: to_dev(a.astype(np.float32))) if storage == "f32" else (
        lambda a: to_dev(bf16_codes(a)))
    if key_values is None:
        kc = rng.standard_normal((B, n_cap, d))
    else:
        kc = key_values[rng.integers(0, len(key_values), size=(B, n_cap))]
    inp = {
        "kc": st(kc), "vc": st(rng.standard_normal((B, n_cap, d))),
        "q": st(rng.standard_normal((B, T, H, d))),
        "qi": st(rng.standard_normal((B, T, H_I, d_I))),
        "w": to_dev(rng.random((B, T, H_I)).astype(np.float32)),
        "pos0": torch.tensor(pos0, dtype=torch.int64, device=DEV),
        "m": m, "W": W, "scale": 1.0 / np.sqrt(d),
    }
    R = W + T + 3
    raw0 = np.asarray(pos0) - (W - 1) - 2
    inp["raw_pos0"] = torch.tensor(raw0, dtype=torch.int64, device=DEV)
    inp["kr"] = st(rng.standard_normal((B, R, d)))
    inp["vr"] = st(rng.standard_normal((B, R, d)))
    inp["zk"] = to_dev(rng.standard_normal((B, R, d)).astype(np.float32))
    inp["zv"] = to_dev(rng.standard_normal((B, R, d)).astype(np.float32))
    inp["ki"], inp["qi_scale"], inp["ki_scale"] = inp["kc"], None, None
    if ki_kind == "fp8":
        inp["qi"], inp["qi_scale"] = csa.csa_quantize_fp8_rows(inp["qi"])
        inp["ki"], inp["ki_scale"] = csa.csa_quantize_fp8_rows(inp["kc"])
    elif ki_kind == "mxfp4":
        inp["qi"], inp["qi_scale"] = csa.csa_quantize_mxfp4_rows(inp["qi"])
        inp["ki"], inp["ki_scale"] = csa.csa_quantize_mxfp4_rows(inp["kc"])
    return inp


def _separate(inp, k):
    sc, idx = csa.csa_index_topk(inp["qi"], inp["w"], inp["ki"], inp["pos0"], inp["m"], k,
                                 qi_scale=inp["qi_scale"], ki_scale=inp["ki_scale"])
    out, lse = csa.csa_attend(inp["q"], inp["kc"], inp["vc"], idx, inp["kr"], inp["vr"],
                              inp["raw_pos0"], inp["pos0"], inp["W"], inp["scale"])
    return sc, idx, out, lse


def _decode(inp, k, ws=None, compress=False):
    return csa.csa_decode(inp["qi"], inp["w"], inp["ki"], inp["q"], inp["kc"], inp["vc"],
                          inp["kr"], inp["vr"], inp["raw_pos0"], inp["pos0"], inp["m"], k,
                          inp["W"], inp["scale"], qi_scale=inp["qi_scale"],
                          ki_scale=inp["ki_scale"], zk=inp["zk"] if compress else None,
                          zv=inp["zv"] if compress else None, ws=ws)


def _same(a, b, what):
    assert a.shape == b.shape, what
    eq = torch.equal(a, b)
    if not eq:
        bad = (a != b).nonzero()[:5].tolist()
        raise AssertionError(f"{what} differs at {bad}")


def _same_scores(a, b, pos0, m, what):
    """Scores agree wherever they are defined (entries j < V(t) of a row)."""
    B, T, n_cap = a.shape
    for bb in range(B):
        for i in range(T):
            V = min(n_cap, (pos0[bb] + i + 1) // m)
            _same(a[bb, i, :V], b[bb, i, :V], f"{what} row ({bb}, {i})")


def _same_all(got, ref, pos0, m, what):
    _same_scores(got[0], ref[0], pos0, m, f"{what} scores")
    for a, b, name in zip(got[1:], ref[1:], ("idx", "out", "lse")):
        _same(a, b, f"{what} {name}")


def _check_oracle_topk(scores, idx, pos0, T, m, k, rows=4):
    s = scores.cpu().numpy().astype(np.float64)
    ix = idx.cpu().numpy()
    B = s.shape[0]
    for b in range(B):
        for i in range(min(T, rows)):
            V = int(oracle.visible_count(np.array([pos0[b] + i]), m)[0])
            V = min(V, s.shape[2])
            assert np.array_equal(ix[b, i], oracle.topk_select(s[b, i], V, k)), (b, i)


CASES = {
    # name: (B, T, n_cap, pos0, k, extra)
    "short_rows_mixed": (4, 1, 3000, [0, 100, 4 * 3000 - 1, 5000], 64, {}),
    "ragged_T2": (3, 2, 5000, [17, 4 * 5000 - 2, 9000], 128, {}),
    "long_rows": (4, 1, 40000, [4 * 40000 - 1, 4 * 33000, 4 * 36001 + 2, 200], 256,
                      {"H": 64, "H_I": 64, "W": 128}),
    "f32_d64": (2, 3, 2048, [8191, 4000], 64, {"storage": "f32", "d": 64, "d_I": 64, "W": 32}),
    "fp8_long": (3, 1, 50000, [4 * 50000 - 1, 4 * 40000, 4 * 20000], 1024,
                 {"ki_kind": "fp8", "H": 64, "H_I": 64, "W": 128}),
    "mxfp4": (2, 1, 33000, [4 * 33000 - 1, 4 * 30000], 512, {"ki_kind": "mxfp4", "H_I": 16}),
    "k_ge_V": (3, 1, 600, [4 * 600 - 1, 300, 3], 1024, {}),
    # rows past 8192 entries take the split top-k, whose selection is made
    # inside the attention launch: rows that keep every visible entry, rows
    # of one slice, ragged T = 2, fp32 at d = 64
    "ragged_T2_long": (3, 2, 20000, [17, 4 * 20000 - 2, 9000], 512,
                       {"H": 64, "H_I": 64, "W": 128}),
    "f32_d64_long": (2, 1, 12000, [4 * 12000 - 1, 30000], 64,
                     {"storage": "f32", "d": 64, "d_I": 64, "W": 32}),
    "bf16_d64_long": (2, 1, 70000, [4 * 70000 - 1, 4 * 9000], 2048,
                      {"d": 64, "d_I": 64, "H": 16, "W": 64}),
    # k not a multiple of the 64-key chunk, no window (W = 0)
    "odd_k_no_window": (3, 1, 20000, [4 * 20000 - 1, 4 * 15000 + 2, 4 * 9000], 1000,
                        {"H": 64, "H_I": 64, "W": 0}),
    # the largest k: lists longer than the attention launch's LDS space
    # (read from global memory)
    "k_max": (2, 1, 70000, [4 * 70000 - 1, 4 * 50000], 4096, {"H": 16, "H_I": 16, "W": 128}),
    # 8 or more rows: the XCD-ordered grids
    "xcd_rows_T2": (5, 2, 12000, [4 * 12000 - 2, 4 * 11000, 4 * 6000, 4 * 3000, 4 * 9999],
                    256, {"H": 32, "H_I": 32, "W": 32}),
    # rows of at most 32768 entries select from registers: every register
    # holding an entry (V = 32768, and 32767), V = k + 1 (every candidate
    # usually wins), a row of one attention split
    # (k + W = 64: the launch itself clears the histogram), and a row
    # length that is no multiple of 4 (the classified lists instead)
    "full_row_regs": (4, 1, 32768, [4 * 32768 - 1, 4 * 32768 - 3, 4 * 20000, 4 * 1025 - 1],
                      1024, {"H": 16, "H_I": 16, "W": 64}),
    "one_split": (2, 1, 12000, [4 * 12000 - 1, 4 * 10000], 48, {"W": 16}),
    "odd_n_cap_lists": (2, 1, 20001, [4 * 20001 - 1, 4 * 15000], 512,
                        {"H": 64, "H_I": 64, "W": 128}),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_decode_matches_separate_calls(name):
    B, T, n_cap, pos0, k, extra = CASES[name]
    say("decode vs separate", name)
    inp = _inputs(sum(map(ord, name)) + 7, B, T, n_cap, pos0, **extra)
    ref = _separate(inp, k)
    ws = csa.workspace(csa.csa_decode_workspace_size(B, T, inp["q"].shape[2], inp["q"].shape[3],
                                                     n_cap, k, inp["W"], False), DEV)
    for call in range(2):  # the second call checks the workspace came back to zero
        got = _decode(inp, k, ws=ws)
        torch.cuda.synchronize()
        _same_all(got, ref, pos0, inp["m"], f"{name} call {call}")
    _check_oracle_topk(got[0], got[1], pos0, T, inp["m"], k)


@pytest.mark.parametrize("name,hist_ready", [("long_rows", True), ("ragged_T2_long", True),
                                              ("fp8_long", True), ("f32_d64_long", False),
                                              ("short_rows_mixed", True), ("one_split", True),
                                              ("full_row_regs", False)])
def test_select_attend_matches_separate_calls(name, hist_ready):
    """csa_select_attend after csa_index_scores (with or without the fused
    histogram) against csa_topk + csa_attend; two calls on one top-k
    workspace, whose histograms must come back to zero."""
    B, T, n_cap, pos0, k, extra = CASES[name]
    say("select_attend vs separate", name, hist_ready)
    inp = _inputs(sum(map(ord, name)) + 11, B, T, n_cap, pos0, **extra)
    ref = _separate(inp, k)
    tws = csa.workspace(csa.csa_topk_workspace_size(B, T, n_cap, k), DEV)
    for call in range(2):
        sc = csa.csa_index_scores(inp["qi"], inp["w"], inp["ki"], inp["pos0"], inp["m"],
                                  qi_scale=inp["qi_scale"], ki_scale=inp["ki_scale"],
                                  topk_ws=tws if hist_ready else None, k=k)
        idx, out, lse = csa.csa_select_attend(sc, tws, inp["pos0"], inp["m"], k, inp["q"],
                                              inp["kc"], inp["vc"], inp["kr"], inp["vr"],
                                              inp["raw_pos0"], inp["W"], inp["scale"],
                                              hist_ready=hist_ready)
        torch.cuda.synchronize()
        _same_all((sc, idx, out, lse), ref, pos0, inp["m"], f"{name} call {call}")
    if tws.numel():
        hist = tws[:B * T * 4096 * 4].view(torch.int32)
        assert int(hist.abs().sum()) == 0


@pytest.mark.parametrize("n_keys,n_cap", [(1, 40000), (3, 40000), (2, 6000), (1, 30000),
                                           (3, 30000), (16, 30000)])
def test_decode_ties(n_keys, n_cap):
    """Keys drawn from n_keys distinct rows: whole rows of equal scores.  One
    distinct key puts every entry in the cut's bucket; the cut then falls
    among equal scores, which go to the lower indices.  At 30000 entries
    (selection from registers) 1 and 3 keys leave more candidates than the
    LDS list holds, 16 keys a list whose cut needs the general digit
    passes."""
    say("ties", n_keys, n_cap)
    rng = np.random.default_rng(n_keys)
    key_values = rng.standard_normal((n_keys, 128))
    B, k = 2, 1024
    pos0 = [4 * n_cap - 1, 4 * (n_cap - 777)]
    inp = _inputs(50 + n_keys, B, 1, n_cap, pos0, key_values=key_values, H=8, H_I=4, W=16)
    ref = _separate(inp, k)
    for rep in range(3):  # several calls: the selection's waves must not race
        got = _decode(inp, k)
        torch.cuda.synchronize()
        _same_all(got, ref, pos0, 4, f"ties {n_keys} call {rep}")
    _check_oracle_topk(got[0], got[1], pos0, 1, 4, k)


def test_decode_block_end_compression():
    """A block-completing token: csa_decode with the compressor logits gives
    the same cache, scores, indices and outputs as csa_decode_index_topk
    followed by csa_attend."""
    say("decode block end")
    B, n_cap, k, W = 4, 9000, 256, 16
    pos0 = [4 * n_cap - 1, 4 * 5000 - 1, 4 * 100 - 1, 4 * 3000 + 1]  # the last one mid-block
    a = _inputs(77, B, 1, n_cap, pos0, W=W)
    b = {key: (v.clone() if isinstance(v, torch.Tensor) else v) for key, v in a.items()}
    b["ki"] = b["kc"]
    sc_r, idx_r = csa.csa_decode_index_topk(a["qi"], a["w"], a["kc"], a["vc"], a["kr"], a["vr"],
                                            a["zk"], a["zv"], a["raw_pos0"], a["pos0"], a["m"], k)
    out_r, lse_r = csa.csa_attend(a["q"], a["kc"], a["vc"], idx_r, a["kr"], a["vr"],
                                  a["raw_pos0"], a["pos0"], W, a["scale"])
    got = _decode(b, k, compress=True)
    torch.cuda.synchronize()
    _same(b["kc"], a["kc"], "kc")
    _same(b["vc"], a["vc"], "vc")
    _same_all(got, (sc_r, idx_r, out_r, lse_r), pos0, 4, "block end")
