"""The kernel-timing hook (csa_time_next_kernels): kernels launched with
their own start / stop events compute exactly what plain launches compute,
the interval they record is positive and no longer than the event pair
around the whole call, and a request is used up by the kernels it names."""

import pytest
import torch

from conftest import ensure_library

ensure_library()
import long_context_sparse_16_amd as csa  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _events():
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    b.record()
    return a, b


def _hca_inputs():
    g = torch.Generator(device="cpu").manual_seed(4100)
    B, T, H, d, m, n_cap, W, R = 2, 1, 64, 128, 128, 1024, 128, 256
    t = n_cap * m - 1  # every entry visible
    bf = lambda *s: torch.randn(*s, generator=g).to(torch.bfloat16).to(DEV)  # noqa: E731
    q, kc, vc = bf(B, T, H, d), bf(B, n_cap, d), bf(B, n_cap, d)
    kr, vr = bf(B, R, d), bf(B, R, d)
    pos0 = torch.full((B,), t, dtype=torch.int64, device=DEV)
    raw_pos0 = pos0 - (R - 1)
    return (q, kc, vc, m, kr, vr, raw_pos0, pos0, W, d ** -0.5)


def test_timed_hca_attention_and_merge():
    args = _hca_inputs()
    assert csa.hca_attend_workspace_size(2, 1, 64, 128, 1024, 128) > 0  # split rows: two kernels
    ref_out, ref_lse = csa.hca_attend(*args)
    a, b = _events()
    c0, c1 = _events()
    c0.record()
    csa.csa_time_next_kernels(a, b, 2)
    out, lse = csa.hca_attend(*args)
    c1.record()
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
    k_ms, call_ms = a.elapsed_time(b), c0.elapsed_time(c1)
    assert 0.0 < k_ms <= call_ms, (k_ms, call_ms)
    # the request was used up: a later call leaves the events alone
    csa.hca_attend(*args)
    torch.cuda.synchronize()
    assert a.elapsed_time(b) == k_ms


def test_timed_indexer_scores():
    g = torch.Generator(device="cpu").manual_seed(4101)
    B, T, H_I, d_I, n_cap, m = 4, 1, 64, 128, 8192, 4
    qi = torch.randn(B, T, H_I, d_I, generator=g).to(torch.bfloat16).to(DEV)
    w = torch.rand(B, T, H_I, generator=g).to(DEV)
    ki = torch.randn(B, n_cap, d_I, generator=g).to(torch.bfloat16).to(DEV)
    pos0 = torch.tensor([n_cap * m - 1, 5000, 17, 20000], dtype=torch.int64, device=DEV)
    ref = csa.csa_index_scores(qi, w, ki, pos0, m)
    a, b = _events()
    csa.csa_time_next_kernels(a, b, 1)
    got = csa.csa_index_scores(qi, w, ki, pos0, m)
    torch.cuda.synchronize()
    for r in range(B):
        V = min(n_cap, (int(pos0[r]) + 1) // m)
        assert torch.equal(got[r, 0, :V], ref[r, 0, :V]), r
    assert a.elapsed_time(b) > 0.0
    csa.csa_time_next_kernels(None, None, 0)
