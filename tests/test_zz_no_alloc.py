"""csa_decode_noalloc (the decode step on the library's fixed per-GPU
scratch, for callers that cannot allocate) against csa_decode with a
workspace: scores, indices, outputs and lse must be bit-identical, since
both run the same kernels.  Calls follow one another on the one scratch:
a larger step, then a smaller one (the scratch keeps the first call's
contents), then a larger one again (its histograms must be re-zeroed where
the smaller call's layout left other data), with the scores kept by the
caller or left in the scratch."""

import pytest
import torch

from conftest import ensure_library
from gpu_util import DEV, say

pytestmark = pytest.mark.gpu

ensure_library()
import long_context_sparse_16_amd as csa  # noqa: E402
import test_gpu_decode as tdec  # noqa: E402


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# (name, B, T, n_cap, pos0, k, extra)
SEQUENCE = [
    ("large", 8, 1, 40000, [4 * 40000 - 1, 4 * 33000, 4 * 36001 + 2, 200, 4 * 39000,
                            4 * 20000 + 3, 4 * 40000 - 5, 4 * 12345], 1024,
     {"H": 64, "H_I": 64, "W": 128}),
    ("smaller", 3, 1, 9000, [4 * 9000 - 1, 4 * 5000, 17], 256, {"H": 16, "H_I": 16, "W": 64}),
    ("ragged_T2", 3, 2, 20000, [17, 4 * 20000 - 2, 9000], 512, {"H": 64, "H_I": 64, "W": 128}),
]


def _run(name, B, T, n_cap, pos0, k, extra, keep_scores):
    inp = tdec._inputs(sum(map(ord, name)) + 3, B, T, n_cap, pos0, **extra)
    ref = tdec._decode(inp, k)
    torch.cuda.synchronize()
    got = csa.csa_decode_noalloc(inp["qi"], inp["w"], inp["ki"], inp["q"], inp["kc"], inp["vc"],
                                 inp["kr"], inp["vr"], inp["raw_pos0"], inp["pos0"], inp["m"], k,
                                 inp["W"], inp["scale"], keep_scores=keep_scores)
    torch.cuda.synchronize()
    if keep_scores:
        tdec._same_scores(got[0], ref[0], pos0, inp["m"], f"{name} scores")
    else:
        assert got[0] is None
    for a, b, what in zip(got[1:], ref[1:], ("idx", "out", "lse")):
        tdec._same(a, b, f"{name} {what}")


@pytest.mark.parametrize("keep_scores", [True, False])
def test_noalloc_matches_workspace_calls(keep_scores):
    assert csa.csa_decode_noalloc_max_bytes() == 64 << 20
    for name, B, T, n_cap, pos0, k, extra in SEQUENCE:
        say("noalloc", name, "keep_scores", keep_scores)
        _run(name, B, T, n_cap, pos0, k, extra, keep_scores)


def test_noalloc_repeated_same_shape():
    """Calls of one size back to back (the steady state of a decode loop):
    no clearing between them, the histograms come back to zero by
    themselves."""
    name, B, T, n_cap, pos0, k, extra = SEQUENCE[0]
    for call in range(3):
        say("noalloc repeat", call)
        _run(name, B, T, n_cap, pos0, k, extra, keep_scores=call == 1)
