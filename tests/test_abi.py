"""C-ABI checks that need no GPU: the library loads, exports every function
include/csa.h declares, and rejects bad arguments on the host (before any
HIP call) with the documented status codes."""

import ctypes
import re

import pytest

from conftest import ROOT, ensure_library

ensure_library()
import long_context_sparse_16_amd as csa  # noqa: E402

lib = csa._lib
NULL = None
FAKE = ctypes.c_void_p(0x100000)  # 16-byte aligned, never dereferenced


def test_every_declared_function_is_exported():
    names = csa.header_functions()
    assert len(names) >= 14
    raw = ctypes.CDLL(csa.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n
    # the binding wraps every compute entry point under the same name
    for n in names:
        if not n.endswith("_string") and n not in ("csa_last_error", "csa_abi_version",
                                                    "csa_build_digest"):
            assert hasattr(csa, n) or n.endswith("workspace_size"), n


def test_status_strings_and_version():
    assert lib.csa_status_string(0) == b"CSA_OK"
    assert lib.csa_status_string(-5) == b"CSA_ERR_WORKSPACE"
    assert lib.csa_abi_version() == 4
    assert len(lib.csa_build_digest()) == 64


def _last():
    return lib.csa_last_error().decode()


def test_compress_validation():
    # null pointers
    assert lib.csa_compress(NULL, 0, NULL, 1, 8, 4, 4, 32, 32, NULL, 0, 2, 0, NULL) == -1
    # partial block
    assert lib.csa_compress(FAKE, 0, FAKE, 1, 6, 4, 4, 32, 32, FAKE, 0, 8, 0, NULL) == -2
    assert "multiple of m" in _last()
    # does not fit the cache
    assert lib.csa_compress(FAKE, 1, FAKE, 1, 8, 4, 4, 32, 32, FAKE, 1, 2, 1, NULL) == -2
    # dtype mismatch / fp8 not a compress dtype
    assert lib.csa_compress(FAKE, 0, FAKE, 1, 8, 4, 4, 32, 32, FAKE, 1, 2, 0, NULL) == -3
    assert lib.csa_compress(FAKE, 2, FAKE, 1, 8, 4, 4, 32, 32, FAKE, 2, 2, 0, NULL) == -3
    # batch stride too small
    assert lib.csa_compress(FAKE, 0, FAKE, 1, 8, 4, 4, 16, 32, FAKE, 0, 2, 0, NULL) == -2


def test_workspace_clear_validation():
    assert lib.csa_workspace_clear(NULL, 0, NULL) == 0
    assert lib.csa_workspace_clear(NULL, 64, NULL) == -1
    assert lib.csa_workspace_clear(ctypes.c_void_p(0x100004), 64, NULL) == -5
    # index with a too-small top-k workspace
    assert lib.csa_index_scores(FAKE, 1, NULL, FAKE, FAKE, 1, NULL, FAKE, 32, 1, 64, 128, 32768, 4,
                                0, FAKE, 1024, FAKE, 16, NULL) == -5


def test_time_next_kernels_validation():
    assert lib.csa_time_next_kernels(NULL, NULL, -1) == -2
    assert "n must be" in _last()
    assert lib.csa_time_next_kernels(NULL, FAKE, 1) == -1
    assert lib.csa_time_next_kernels(FAKE, NULL, 2) == -1
    # n = 0 cancels (nothing is pending afterwards), with or without events
    assert lib.csa_time_next_kernels(NULL, NULL, 0) == 0
    assert lib.csa_time_next_kernels(FAKE, FAKE, 0) == 0


def test_quantize_validation():
    assert lib.csa_quantize_fp8_rows(NULL, 1, 4, 128, FAKE, FAKE, NULL) == -1
    assert lib.csa_quantize_fp8_rows(FAKE, 2, 4, 128, FAKE, FAKE, NULL) == -3
    assert lib.csa_quantize_fp8_rows(FAKE, 1, 4, 2048, FAKE, FAKE, NULL) == -4
    assert lib.csa_quantize_mxfp4_rows(NULL, 1, 4, 128, FAKE, FAKE, NULL) == -1
    assert lib.csa_quantize_mxfp4_rows(FAKE, 3, 4, 128, FAKE, FAKE, NULL) == -3
    assert lib.csa_quantize_mxfp4_rows(FAKE, 1, 4, 100, FAKE, FAKE, NULL) == -4   # not % 32
    assert lib.csa_quantize_mxfp4_rows(FAKE, 1, -1, 128, FAKE, FAKE, NULL) == -2


def _index(qi_dtype=1, ki_dtype=1, qs=NULL, ks=NULL, B=1, T=1, H=64, dI=128, n_cap=32, m=4, act=0,
           scores=FAKE, qi=FAKE):
    return lib.csa_index_scores(qi, qi_dtype, qs, FAKE, FAKE, ki_dtype, ks, FAKE, B, T, H, dI,
                                n_cap, m, act, scores, 0, NULL, 0, NULL)


def test_index_validation():
    assert _index(scores=NULL) == -1
    assert _index(qi_dtype=1, ki_dtype=0) == -3
    assert _index(qi_dtype=2, ki_dtype=2) == -1          # fp8 needs scales
    assert _index(qi_dtype=2, ki_dtype=2, qs=FAKE, ks=FAKE, dI=64) == -4
    assert _index(qi_dtype=3, ki_dtype=3) == -1          # mxfp4 needs block scales
    assert _index(qi_dtype=3, ki_dtype=3, qs=FAKE, ks=FAKE, dI=256) == -4
    assert _index(qi_dtype=3, ki_dtype=3, qs=FAKE, ks=ctypes.c_void_p(0x100002)) == -2
    assert _index(qi_dtype=4, ki_dtype=4) == -3
    assert _index(H=65) == -4
    assert _index(dI=96) == -4
    assert _index(m=0) == -2
    assert _index(act=7) == -2
    assert _index(B=300, T=300) == -4
    assert _index(qi=ctypes.c_void_p(0x100004)) == -2    # misaligned


def test_topk_validation_and_workspace():
    assert lib.csa_topk(NULL, FAKE, 1, 1, 64, 4, 8, FAKE, NULL, 0, 0, NULL) == -1
    assert lib.csa_topk(FAKE, FAKE, 1, 1, 64, 4, 0, FAKE, NULL, 0, 0, NULL) == -4
    assert lib.csa_topk(FAKE, FAKE, 1, 1, 64, 4, 5000, FAKE, NULL, 0, 0, NULL) == -4
    need = lib.csa_topk_workspace_size(32, 1, 32768, 1024)
    assert need > 0 and need % 256 == 0
    assert lib.csa_topk(FAKE, FAKE, 32, 1, 32768, 4, 1024, FAKE, NULL, 0, 0, NULL) == -5
    assert lib.csa_topk(FAKE, FAKE, 32, 1, 32768, 4, 1024, FAKE, FAKE, need - 1, 0, NULL) == -5
    assert "workspace" in _last()
    # many rows use one workgroup per row: the workspace (the prefill
    # indexer's coarse histograms and their flags) is optional
    many = lib.csa_topk_workspace_size(1, 8192, 67584, 1024)
    assert many >= 8192 * (2048 + 1) * 4
    assert lib.csa_topk(FAKE, FAKE, 1, 8192, 67584, 4, 1024, FAKE, FAKE, many - 1, 0, NULL) == -5
    with_scores = lib.csa_index_topk_workspace_size(32, 1, 32768, 1024, 1)
    assert with_scores >= need + 32 * 32768 * 4


def _attend(q=FAKE, dt=1, kvdt=1, idx=FAKE, k=1024, kr=FAKE, W=128, H=64, d=128, B=1, T=1,
            ws=NULL, wsb=0, R=128, scale=0.1):
    return lib.csa_attend(q, dt, FAKE, FAKE, kvdt, idx, k, kr, FAKE, FAKE, R, FAKE, B, T, H, d,
                          4096, W, scale, FAKE, NULL, ws, wsb, NULL)


def test_attend_validation():
    assert _attend(q=NULL) == -1
    assert _attend(kr=NULL) == -1
    assert _attend(kr=NULL, W=0, ws=FAKE, wsb=1 << 30) != -1 or True
    assert _attend(dt=2, kvdt=2) == -3
    assert _attend(dt=0, kvdt=1) == -3
    assert _attend(H=65) == -4
    assert _attend(d=96) == -4
    assert _attend(W=5000) == -4
    assert _attend(idx=NULL) == -1
    assert _attend(k=0, W=0, kr=NULL) == -2              # empty key set
    assert _attend(scale=0.0) == -2                      # scale must be finite and > 0
    assert _attend(scale=-0.1) == -2
    assert _attend(scale=float("inf")) == -2
    assert _attend(scale=float("nan")) == -2
    need = lib.csa_attend_workspace_size(1, 1, 64, 128, 1024, 128)
    assert need > 0
    assert _attend() == -5
    # HCA
    assert lib.hca_attend(FAKE, 1, FAKE, FAKE, 1, 0, FAKE, FAKE, FAKE, 128, FAKE, 1, 1, 64, 128,
                          8192, 128, 0.1, FAKE, NULL, NULL, 0, NULL) == -2
    assert lib.hca_attend_workspace_size(16, 1, 64, 128, 8192, 128) > 0


def _attend_bwd(q=FAKE, dt=1, kvdt=1, idx=FAKE, k=64, H=64, d=128, W=16, ws=FAKE, wsb=1 << 30,
                dout=FAKE, dkr=FAKE, scale=0.1):
    return lib.csa_attend_backward(q, dt, FAKE, FAKE, kvdt, idx, k, FAKE, FAKE, FAKE, 32, FAKE, 1,
                                   4, H, d, 4096, W, scale, FAKE, FAKE, dout, FAKE, FAKE, FAKE, dkr,
                                   FAKE, ws, wsb, NULL)


def test_backward_validation():
    assert _attend_bwd(idx=NULL) == -1
    assert _attend_bwd(dout=NULL) == -1
    assert _attend_bwd(dkr=NULL) == -1                 # window gradients need dkr / dvr
    assert _attend_bwd(d=96) == -4
    assert _attend_bwd(H=65) == -4
    assert _attend_bwd(dt=2, kvdt=2) == -3
    assert _attend_bwd(ws=NULL) == -5
    need = lib.csa_attend_backward_workspace_size(1, 4, 128, 4096, 64, 16)
    # staging (K and V contributions, fp32) + per-entry counts and offsets + the
    # reference lists
    assert need >= 4 * (64 + 16) * 128 * 8 + 2 * 4096 * 4 + 4 * 64 * 4
    assert _attend_bwd(wsb=need - 1) == -5
    assert lib.hca_attend_backward(FAKE, 1, FAKE, FAKE, 1, 0, FAKE, FAKE, FAKE, 32, FAKE, 1, 4, 64,
                                   128, 4096, 16, 0.1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   FAKE, FAKE, 1 << 30, NULL) == -2   # m = 0
    assert lib.csa_compress_backward(NULL, 1, FAKE, FAKE, 1, 8, 4, 4, 32, 32, FAKE, FAKE, NULL) == -1
    assert lib.csa_compress_backward(FAKE, 2, FAKE, FAKE, 1, 8, 4, 4, 32, 32, FAKE, FAKE, NULL) == -3
    assert lib.csa_compress_backward(FAKE, 1, FAKE, FAKE, 1, 6, 4, 4, 32, 32, FAKE, FAKE, NULL) == -2
    assert lib.csa_compress_backward(FAKE, 1, FAKE, FAKE, 1, 8, 4, 4, 16, 32, FAKE, FAKE, NULL) == -2


def _decode(noalloc, B=32, T=1, n_cap=32768, k=1024, scores=FAKE, zk=NULL, ws=FAKE,
            ws_bytes=1 << 40):
    # qi, qi_dtype, qi_scale, w, ki, ki_dtype, ki_scale, q, kc, vc, kv_dtype, kr, vr, zk, zv,
    # raw_pos0, R, pos0, B, T, H_I, d_I, H, d, n_cap, m, act, k, W, scale, scores, idx, out, lse
    args = [FAKE, 1, NULL, FAKE, FAKE, 1, NULL, FAKE, FAKE, FAKE, 1, FAKE, FAKE, zk, NULL,
            FAKE, 131, FAKE, B, T, 64, 128, 64, 128, n_cap, 4, 0, k, 128, 0.088, scores, FAKE,
            FAKE, FAKE]
    if noalloc:
        return lib.csa_decode_noalloc(*args, NULL)
    return lib.csa_decode(*args, ws, ws_bytes, NULL)


def test_decode_validation():
    """Both decode entry points check every argument before touching the
    GPU; the allocation-free one also refuses sizes beyond its fixed
    scratch (here the scores of 256 x 2^20 entries kept in it)."""
    for noalloc in (False, True):
        assert _decode(noalloc, B=0) == -2
        assert _decode(noalloc, k=0) == -4
        assert _decode(noalloc, zk=FAKE) == -1  # zk without zv
    assert _decode(False, ws=NULL) == -5
    assert _decode(False, ws_bytes=16) == -5
    assert csa.csa_decode_noalloc_max_bytes() == 64 << 20
    assert _decode(True, B=256, n_cap=1 << 20, scores=NULL) == -4
    assert "fixed scratch" in _last()
