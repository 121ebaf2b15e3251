"""Python binding of libcsa.so, the C ABI declared in include/csa.h.

Argument marshalling only: every function takes PyTorch tensors (device
memory) and passes their data pointers, sizes and the current HIP stream to
the library entry point of the same name.  All computation happens in the
HIP kernels; there is no fallback path.  Importing this module fails if the
library has not been built (``python long_context_sparse_16_amd/build.py``).

Output tensors and workspaces that are not supplied are allocated with
PyTorch on the inputs' device.
"""

from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "csa.h")

CSA_F32, CSA_BF16, CSA_FP8_E4M3, CSA_MXFP4 = 0, 1, 2, 3
CSA_ACT_RELU, CSA_ACT_IDENTITY = 0, 1


class CSAError(RuntimeError):
    """A library call returned a non-zero status."""

    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed with {status} ({_status_name(status)}): {message}")
        self.status = status


if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library first "
        "(python long_context_sparse_16_amd/build.py)")

_lib = ctypes.CDLL(LIB_PATH)

_vp, _i, _i64, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t

_SIGNATURES = {
    "csa_status_string": (ctypes.c_char_p, [_i]),
    "csa_last_error": (ctypes.c_char_p, []),
    "csa_abi_version": (_i, []),
    "csa_build_digest": (ctypes.c_char_p, []),
    "csa_workspace_clear": (_i, [_vp, _sz, _vp]),
    "csa_time_next_kernels": (_i, [_vp, _vp, _i]),
    "csa_compress": (_i, [_vp, _i, _vp, _i64, _i64, _i64, _i, _i64, _i64, _vp, _i, _i64, _i64, _vp]),
    "csa_quantize_fp8_rows": (_i, [_vp, _i, _i64, _i64, _vp, _vp, _vp]),
    "csa_quantize_mxfp4_rows": (_i, [_vp, _i, _i64, _i64, _vp, _vp, _vp]),
    "csa_index_scores": (_i, [_vp, _i, _vp, _vp, _vp, _i, _vp, _vp, _i64, _i64, _i64, _i64, _i64,
                              _i, _i, _vp, _i, _vp, _sz, _vp]),
    "csa_topk_workspace_size": (_sz, [_i64, _i64, _i64, _i]),
    "csa_topk": (_i, [_vp, _vp, _i64, _i64, _i64, _i, _i, _vp, _vp, _sz, _i, _vp]),
    "csa_index_topk_workspace_size": (_sz, [_i64, _i64, _i64, _i, _i]),
    "csa_index_topk": (_i, [_vp, _i, _vp, _vp, _vp, _i, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i,
                            _i, _i, _vp, _vp, _vp, _sz, _vp]),
    "csa_decode_index_topk": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _i64,
                                   _i64, _i64, _i64, _i, _i, _i, _vp, _vp, _vp, _sz, _vp]),
    "csa_attend_workspace_size": (_sz, [_i64, _i64, _i64, _i64, _i, _i]),
    "csa_select_attend": (_i, [_vp, _vp, _sz, _i, _vp, _i, _i, _vp, _vp, _vp, _i, _vp, _vp,
                               _vp, _i64, _i64, _i64, _i64, _i64, _i64, _i, _f, _vp, _vp, _vp,
                               _vp, _sz, _vp]),
    "csa_decode_workspace_size": (_sz, [_i64, _i64, _i64, _i64, _i64, _i, _i, _i]),
    "csa_decode_noalloc_max_bytes": (_sz, []),
    "csa_decode_noalloc": (_i, [_vp, _i, _vp, _vp, _vp, _i, _vp, _vp, _vp, _vp, _i, _vp, _vp,
                                _vp, _vp, _vp, _i64, _vp, _i64, _i64, _i64, _i64, _i64, _i64,
                                _i64, _i, _i, _i, _i, _f, _vp, _vp, _vp, _vp, _vp]),
    "csa_decode": (_i, [_vp, _i, _vp, _vp, _vp, _i, _vp, _vp, _vp, _vp, _i, _vp, _vp, _vp, _vp,
                        _vp, _i64, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i, _i, _i, _i,
                        _f, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "csa_attend": (_i, [_vp, _i, _vp, _vp, _i, _vp, _i, _vp, _vp, _vp, _i64, _vp, _i64, _i64, _i64,
                        _i64, _i64, _i, _f, _vp, _vp, _vp, _sz, _vp]),
    "hca_attend_workspace_size": (_sz, [_i64, _i64, _i64, _i64, _i64, _i]),
    "csa_attend_backward_workspace_size": (_sz, [_i64, _i64, _i64, _i64, _i, _i]),
    "csa_attend_backward": (_i, [_vp, _i, _vp, _vp, _i, _vp, _i, _vp, _vp, _vp, _i64, _vp, _i64,
                                 _i64, _i64, _i64, _i64, _i, _f, _vp, _vp, _vp, _vp, _vp, _vp,
                                 _vp, _vp, _vp, _sz, _vp]),
    "hca_attend_backward_workspace_size": (_sz, [_i64, _i64, _i64, _i64, _i]),
    "hca_attend_backward": (_i, [_vp, _i, _vp, _vp, _i, _i, _vp, _vp, _vp, _i64, _vp, _i64, _i64,
                                 _i64, _i64, _i64, _i, _f, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                 _vp, _vp, _sz, _vp]),
    "csa_compress_backward": (_i, [_vp, _i, _vp, _vp, _i64, _i64, _i64, _i, _i64, _i64, _vp, _vp,
                                   _vp]),
    "hca_attend": (_i, [_vp, _i, _vp, _vp, _i, _i, _vp, _vp, _vp, _i64, _vp, _i64, _i64, _i64, _i64,
                        _i64, _i, _f, _vp, _vp, _vp, _sz, _vp]),
}

for _name, (_res, _args) in _SIGNATURES.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


def _source_digest() -> str:
    import importlib.util
    spec = importlib.util.spec_from_file_location("_csa_build", os.path.join(_HERE, "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.source_digest()


if _lib.csa_build_digest().decode() != _source_digest():
    raise ImportError(
        f"{LIB_PATH} was built from other sources than the ones in this tree: rebuild it "
        "(python long_context_sparse_16_amd/build.py)")


def header_functions() -> list:
    """Names of the functions declared in include/csa.h."""
    with open(HEADER_PATH) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    return sorted(set(re.findall(r"\b(csa_\w+|hca_\w+)\s*\(", text)))


def _status_name(status: int) -> str:
    return _lib.csa_status_string(status).decode()


def last_error() -> str:
    return _lib.csa_last_error().decode()


def abi_version() -> int:
    return _lib.csa_abi_version()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise CSAError(fn, status, last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return CSA_F32
    if t.dtype == torch.bfloat16:
        return CSA_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return CSA_FP8_E4M3
    if t.dtype == torch.float4_e2m1fn_x2:
        return CSA_MXFP4
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream, device) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("all tensors must be on a HIP device")
            return t.device
    raise ValueError("no tensor given")


def _contig(name: str, t: torch.Tensor) -> None:
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _act_code(act) -> int:
    if act in ("relu", CSA_ACT_RELU):
        return CSA_ACT_RELU
    if act in ("identity", CSA_ACT_IDENTITY):
        return CSA_ACT_IDENTITY
    raise ValueError(f"unknown act {act!r}")


# ----------------------------------------------------------------- compress

def csa_compress(x: torch.Tensor, logits: torch.Tensor, cache: torch.Tensor, m: int,
                 first_entry: int = 0, stream=None) -> torch.Tensor:
    """Append compressed entries to ``cache`` [B, n_cap, d].

    x: [B, n_tok, d] (rows contiguous; the batch stride may be larger, e.g.
    a slice of a longer raw buffer), logits: [B, n_tok, d] float32 likewise.
    Writes entries first_entry .. first_entry + n_tok/m - 1; returns cache.
    """
    dev = _dev(x, logits, cache)
    B, n_tok, d = x.shape
    for name, t in (("x", x), ("logits", logits)):
        if t.shape != (B, n_tok, d) or t.stride(2) != 1 or (n_tok > 1 and t.stride(1) != d):
            raise ValueError(f"{name} must be [B, n_tok, d] with contiguous rows")
    if logits.dtype != torch.float32:
        raise TypeError("logits must be float32")
    _contig("cache", cache)
    if cache.dim() != 3 or cache.shape[0] != B or cache.shape[2] != d:
        raise ValueError("cache must be [B, n_cap, d]")
    _check("csa_compress", _lib.csa_compress(
        _ptr(x), _dtype_code(x), _ptr(logits), B, n_tok, d, int(m), x.stride(0), logits.stride(0),
        _ptr(cache), _dtype_code(cache), cache.shape[1], int(first_entry), _stream(stream, dev)))
    return cache


def csa_quantize_fp8_rows(x: torch.Tensor, codes: torch.Tensor = None, scales: torch.Tensor = None,
                          stream=None):
    """Quantize the rows (last axis) of x to E4M3 codes (uint8) plus one fp32
    scale per row.  Returns (codes, scales) shaped like x and x.shape[:-1]."""
    dev = _dev(x)
    _contig("x", x)
    d = x.shape[-1]
    rows = x.numel() // d if d else 0
    if codes is None:
        codes = torch.empty(x.shape, dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty(x.shape[:-1], dtype=torch.float32, device=dev)
    _contig("codes", codes)
    _contig("scales", scales)
    if codes.numel() != x.numel() or scales.numel() != rows:
        raise ValueError("codes / scales have the wrong size")
    _check("csa_quantize_fp8_rows", _lib.csa_quantize_fp8_rows(
        _ptr(x), _dtype_code(x), rows, d, _ptr(codes), _ptr(scales), _stream(stream, dev)))
    return codes, scales


def csa_quantize_mxfp4_rows(x: torch.Tensor, codes: torch.Tensor = None,
                            scales: torch.Tensor = None, stream=None):
    """Quantize the rows (last axis, a multiple of 32) of x to MXFP4.
    Returns (codes, scales): codes torch.float4_e2m1fn_x2 [..., d/2] (two
    E2M1 codes per byte, low nibble first), scales torch.float8_e8m0fnu
    [..., d/32] (one per 32-element block)."""
    dev = _dev(x)
    _contig("x", x)
    d = x.shape[-1]
    rows = x.numel() // d if d else 0
    if codes is None:
        codes = torch.empty(x.shape[:-1] + (d // 2,), dtype=torch.uint8,
                            device=dev).view(torch.float4_e2m1fn_x2)
    if scales is None:
        scales = torch.empty(x.shape[:-1] + (d // 32,), dtype=torch.uint8,
                             device=dev).view(torch.float8_e8m0fnu)
    _contig("codes", codes)
    _contig("scales", scales)
    if codes.numel() * 2 != x.numel() or scales.numel() * 32 != x.numel():
        raise ValueError("codes / scales have the wrong size")
    _check("csa_quantize_mxfp4_rows", _lib.csa_quantize_mxfp4_rows(
        _ptr(x), _dtype_code(x), rows, d, _ptr(codes), _ptr(scales), _stream(stream, dev)))
    return codes, scales


# ------------------------------------------------------------------ indexer

def _index_shapes(qi, w, ki, pos0):
    """Shapes of the indexer operands; for MXFP4 (float4_e2m1fn_x2) the last
    axis holds d_I / 2 bytes."""
    if qi.dim() != 4:
        raise ValueError("qi must be [B, T, H_I, d_I]")
    B, T, H_I, d_I = qi.shape
    if qi.dtype == torch.float4_e2m1fn_x2:
        d_I *= 2
    if ki.dim() != 3 or ki.shape[0] != B or ki.shape[2] != qi.shape[3]:
        raise ValueError("ki must be [B, n_cap, d_I]")
    if w.shape != (B, T, H_I) or w.dtype != torch.float32:
        raise ValueError("w must be float32 [B, T, H_I]")
    if pos0.shape != (B,) or pos0.dtype != torch.int64:
        raise ValueError("pos0 must be int64 [B]")
    for name, t in (("qi", qi), ("w", w), ("ki", ki), ("pos0", pos0)):
        _contig(name, t)
    return B, T, H_I, d_I, ki.shape[1]


def csa_index_scores(qi, w, ki, pos0, m: int, act="relu", qi_scale=None, ki_scale=None,
                     scores=None, topk_ws=None, k: int = 0, stream=None) -> torch.Tensor:
    """Lightning Indexer scores [B, T, n_cap] (entries j >= V(t) untouched).

    With ``topk_ws`` (a clean top-k workspace) and ``k``, the first-digit
    histogram of the top-k is built on the way; follow with
    ``csa_topk(..., ws=topk_ws, hist_ready=True)``."""
    dev = _dev(qi, w, ki, pos0)
    B, T, H_I, d_I, n_cap = _index_shapes(qi, w, ki, pos0)
    if scores is None:
        scores = torch.empty((B, T, n_cap), dtype=torch.float32, device=dev)
    _contig("scores", scores)
    if scores.shape != (B, T, n_cap) or scores.dtype != torch.float32:
        raise ValueError("scores must be float32 [B, T, n_cap]")
    nbytes = 0 if topk_ws is None else topk_ws.numel() * topk_ws.element_size()
    _check("csa_index_scores", _lib.csa_index_scores(
        _ptr(qi), _dtype_code(qi), _ptr(qi_scale), _ptr(w), _ptr(ki), _dtype_code(ki),
        _ptr(ki_scale), _ptr(pos0), B, T, H_I, d_I, n_cap, int(m), _act_code(act), _ptr(scores),
        int(k), _ptr(topk_ws), nbytes, _stream(stream, dev)))
    return scores


def csa_topk_workspace_size(B: int, T: int, n_cap: int, k: int) -> int:
    return int(_lib.csa_topk_workspace_size(B, T, n_cap, k))


def workspace(nbytes: int, device) -> torch.Tensor:
    """A zero-filled workspace (the state every call expects and leaves)."""
    return torch.zeros(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def csa_workspace_clear(ws: torch.Tensor, stream=None) -> None:
    _check("csa_workspace_clear", _lib.csa_workspace_clear(
        _ptr(ws), ws.numel() * ws.element_size() // 4 * 4, _stream(stream, ws.device)))


def csa_time_next_kernels(start_event, stop_event, n: int) -> None:
    """Record start_event when the next library kernel starts and stop_event
    when the n-th ends (torch.cuda.Event objects with enable_timing, already
    recorded once so that their HIP events exist, or raw hipEvent_t values);
    n = 0 cancels."""
    def handle(e):
        if e is None:
            return None
        return ctypes.c_void_p(e.cuda_event if hasattr(e, "cuda_event") else int(e))
    _check("csa_time_next_kernels",
           _lib.csa_time_next_kernels(handle(start_event), handle(stop_event), int(n)))


def _workspace(ws, need, dev):
    if need == 0:
        return ws, 0 if ws is None else ws.numel() * ws.element_size()
    if ws is None:
        ws = workspace(need, dev)
    if ws.numel() * ws.element_size() < need:
        raise ValueError(f"workspace needs {need} bytes")
    return ws, ws.numel() * ws.element_size()


def csa_topk(scores, pos0, m: int, k: int, idx=None, ws=None, hist_ready=False,
             stream=None) -> torch.Tensor:
    """Top-k entry indices [B, T, k] int32, ascending, padded with -1."""
    dev = _dev(scores, pos0)
    _contig("scores", scores)
    B, T, n_cap = scores.shape
    if idx is None:
        idx = torch.empty((B, T, k), dtype=torch.int32, device=dev)
    _contig("idx", idx)
    ws, nbytes = _workspace(ws, csa_topk_workspace_size(B, T, n_cap, k), dev)
    _check("csa_topk", _lib.csa_topk(
        _ptr(scores), _ptr(pos0), B, T, n_cap, int(m), int(k), _ptr(idx), _ptr(ws), nbytes,
        int(bool(hist_ready)), _stream(stream, dev)))
    return idx


def csa_index_topk_workspace_size(B: int, T: int, n_cap: int, k: int,
                                  scores_in_workspace: bool) -> int:
    return int(_lib.csa_index_topk_workspace_size(B, T, n_cap, k, int(bool(scores_in_workspace))))


def csa_index_topk(qi, w, ki, pos0, m: int, k: int, act="relu", qi_scale=None, ki_scale=None,
                   scores=None, idx=None, ws=None, keep_scores=True, stream=None):
    """Indexer scores followed by top-k.  Returns (scores or None, idx)."""
    dev = _dev(qi, w, ki, pos0)
    B, T, H_I, d_I, n_cap = _index_shapes(qi, w, ki, pos0)
    if scores is None and keep_scores:
        scores = torch.empty((B, T, n_cap), dtype=torch.float32, device=dev)
    if idx is None:
        idx = torch.empty((B, T, k), dtype=torch.int32, device=dev)
    ws, nbytes = _workspace(ws, csa_index_topk_workspace_size(B, T, n_cap, k, scores is None), dev)
    _check("csa_index_topk", _lib.csa_index_topk(
        _ptr(qi), _dtype_code(qi), _ptr(qi_scale), _ptr(w), _ptr(ki), _dtype_code(ki),
        _ptr(ki_scale), _ptr(pos0), B, T, H_I, d_I, n_cap, int(m), _act_code(act), int(k),
        _ptr(scores), _ptr(idx), _ptr(ws), nbytes, _stream(stream, dev)))
    return scores, idx


def csa_decode_index_topk(qi, w, kc, vc, kr, vr, zk, zv, raw_pos0, pos0, m: int, k: int,
                          act="relu", scores=None, idx=None, ws=None, keep_scores=True,
                          stream=None):
    """Decode step selection with the block compression fused into the
    indexer: when a query's position t completes a block, entry
    (t + 1) / m - 1 of kc / vc is formed from the raw rows first (as
    csa_compress would), then indexer scores and top-k as csa_index_topk
    with ki = kc.  qi [B, 1, H_I, d] bf16, w [B, 1, H_I], kr / vr [B, R, d]
    bf16, zk / zv [B, R, d] fp32.  Returns (scores or None, idx)."""
    dev = _dev(qi, w, kc, pos0)
    B, T, H_I, d, n_cap = _index_shapes(qi, w, kc, pos0)
    if T != 1:
        raise ValueError("one query token per sequence (qi [B, 1, H_I, d])")
    for name, t in (("qi", qi), ("kc", kc), ("vc", vc), ("kr", kr), ("vr", vr)):
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bfloat16")
    if vc.shape != kc.shape:
        raise ValueError("vc must have kc's shape")
    if kr.dim() != 3 or kr.shape[0] != B or kr.shape[2] != d or vr.shape != kr.shape:
        raise ValueError("kr, vr must be [B, R, d]")
    for name, t in (("zk", zk), ("zv", zv)):
        if t.shape != kr.shape or t.dtype != torch.float32:
            raise ValueError(f"{name} must be float32 [B, R, d]")
    if raw_pos0.shape != (B,) or raw_pos0.dtype != torch.int64:
        raise ValueError("raw_pos0 must be int64 [B]")
    for name, t in (("vc", vc), ("kr", kr), ("vr", vr), ("zk", zk), ("zv", zv),
                    ("raw_pos0", raw_pos0)):
        _contig(name, t)
    if scores is None and keep_scores:
        scores = torch.empty((B, 1, n_cap), dtype=torch.float32, device=dev)
    if idx is None:
        idx = torch.empty((B, 1, k), dtype=torch.int32, device=dev)
    ws, nbytes = _workspace(ws, csa_index_topk_workspace_size(B, 1, n_cap, k, scores is None), dev)
    _check("csa_decode_index_topk", _lib.csa_decode_index_topk(
        _ptr(qi), _ptr(w), _ptr(kc), _ptr(vc), _ptr(kr), _ptr(vr), _ptr(zk), _ptr(zv),
        _ptr(raw_pos0), kr.shape[1], _ptr(pos0), B, H_I, d, n_cap, int(m), _act_code(act), int(k),
        _ptr(scores), _ptr(idx), _ptr(ws), nbytes, _stream(stream, dev)))
    return scores, idx


# ---------------------------------------------------------------- attention

def _attend_shapes(q, kc, vc, kr, vr, raw_pos0, pos0, W):
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, d]")
    B, T, H, d = q.shape
    if kc.dim() != 3 or kc.shape[0] != B or kc.shape[2] != d or vc.shape != kc.shape:
        raise ValueError("kc, vc must be [B, n_cap, d]")
    R = 0
    if W > 0:
        if kr.dim() != 3 or kr.shape[0] != B or kr.shape[2] != d or vr.shape != kr.shape:
            raise ValueError("kr, vr must be [B, R, d]")
        R = kr.shape[1]
        if raw_pos0.shape != (B,) or raw_pos0.dtype != torch.int64:
            raise ValueError("raw_pos0 must be int64 [B]")
    if pos0.shape != (B,) or pos0.dtype != torch.int64:
        raise ValueError("pos0 must be int64 [B]")
    for name, t in (("q", q), ("kc", kc), ("vc", vc), ("kr", kr), ("vr", vr),
                    ("raw_pos0", raw_pos0), ("pos0", pos0)):
        if t is not None:
            _contig(name, t)
    return B, T, H, d, kc.shape[1], R


def _outputs(out, lse, B, T, H, d, dev, want_lse):
    if out is None:
        out = torch.empty((B, T, H, d), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    _contig("out", out)
    if out.shape != (B, T, H, d) or out.dtype != torch.float32:
        raise ValueError("out must be float32 [B, T, H, d]")
    if lse is not None and (lse.shape != (B, T, H) or lse.dtype != torch.float32):
        raise ValueError("lse must be float32 [B, T, H]")
    return out, lse


def csa_attend_workspace_size(B, T, H, d, k, W) -> int:
    return int(_lib.csa_attend_workspace_size(B, T, H, d, k, W))


def csa_attend(q, kc, vc, idx, kr, vr, raw_pos0, pos0, W: int, scale: float, out=None, lse=None,
               want_lse=True, ws=None, stream=None):
    """Attention over the selected entries plus the window.  Returns (out, lse)."""
    dev = _dev(q, kc, vc, pos0)
    B, T, H, d, n_cap, R = _attend_shapes(q, kc, vc, kr, vr, raw_pos0, pos0, W)
    k = 0
    if idx is not None:
        _contig("idx", idx)
        if idx.dim() != 3 or idx.shape[:2] != (B, T) or idx.dtype != torch.int32:
            raise ValueError("idx must be int32 [B, T, k]")
        k = idx.shape[2]
    out, lse = _outputs(out, lse, B, T, H, d, dev, want_lse)
    ws, nbytes = _workspace(ws, csa_attend_workspace_size(B, T, H, d, k, W), dev)
    _check("csa_attend", _lib.csa_attend(
        _ptr(q), _dtype_code(q), _ptr(kc), _ptr(vc), _dtype_code(kc), _ptr(idx), k, _ptr(kr),
        _ptr(vr), _ptr(raw_pos0), R, _ptr(pos0), B, T, H, d, n_cap, int(W), float(scale),
        _ptr(out), _ptr(lse), _ptr(ws), nbytes, _stream(stream, dev)))
    return out, lse


def hca_attend_workspace_size(B, T, H, d, n_cap, W) -> int:
    return int(_lib.hca_attend_workspace_size(B, T, H, d, n_cap, W))


def hca_attend(q, kc, vc, m: int, kr, vr, raw_pos0, pos0, W: int, scale: float, out=None,
               lse=None, want_lse=True, ws=None, stream=None):
    """Dense attention over all visible compressed entries plus the window."""
    dev = _dev(q, kc, vc, pos0)
    B, T, H, d, n_cap, R = _attend_shapes(q, kc, vc, kr, vr, raw_pos0, pos0, W)
    out, lse = _outputs(out, lse, B, T, H, d, dev, want_lse)
    ws, nbytes = _workspace(ws, hca_attend_workspace_size(B, T, H, d, n_cap, W), dev)
    _check("hca_attend", _lib.hca_attend(
        _ptr(q), _dtype_code(q), _ptr(kc), _ptr(vc), _dtype_code(kc), int(m), _ptr(kr), _ptr(vr),
        _ptr(raw_pos0), R, _ptr(pos0), B, T, H, d, n_cap, int(W), float(scale), _ptr(out),
        _ptr(lse), _ptr(ws), nbytes, _stream(stream, dev)))
    return out, lse


# ------------------------------------------------------------- backward pass

# -------------------------------------------------------------- decode step

def csa_select_attend(scores, topk_ws, pos0, m: int, k: int, q, kc, vc, kr, vr, raw_pos0,
                      W: int, scale: float, hist_ready=True, idx=None, out=None, lse=None,
                      want_lse=True, ws=None, stream=None):
    """Top-k selection (from csa_index_scores' scores and, with hist_ready,
    the histogram it built in topk_ws) and attention over the selection.
    Returns (idx, out, lse)."""
    dev = _dev(scores, q, kc, pos0)
    B, T, H, d, n_cap, R = _attend_shapes(q, kc, vc, kr, vr, raw_pos0, pos0, W)
    _contig("scores", scores)
    if scores.shape != (B, T, n_cap) or scores.dtype != torch.float32:
        raise ValueError("scores must be float32 [B, T, n_cap]")
    if idx is None:
        idx = torch.empty((B, T, k), dtype=torch.int32, device=dev)
    out, lse = _outputs(out, lse, B, T, H, d, dev, want_lse)
    ws, nbytes = _workspace(ws, csa_attend_workspace_size(B, T, H, d, k, W), dev)
    tws_bytes = topk_ws.numel() * topk_ws.element_size() if topk_ws is not None else 0
    _check("csa_select_attend", _lib.csa_select_attend(
        _ptr(scores), _ptr(topk_ws), tws_bytes, int(bool(hist_ready)), _ptr(pos0), int(m),
        int(k), _ptr(q), _ptr(kc), _ptr(vc), _dtype_code(kc), _ptr(kr), _ptr(vr),
        _ptr(raw_pos0), R, B, T, H, d, n_cap, int(W), float(scale), _ptr(idx), _ptr(out),
        _ptr(lse), _ptr(ws), nbytes, _stream(stream, dev)))
    return idx, out, lse


def csa_decode_workspace_size(B: int, T: int, H: int, d: int, n_cap: int, k: int, W: int,
                              scores_in_workspace: bool) -> int:
    return int(_lib.csa_decode_workspace_size(B, T, H, d, n_cap, k, W,
                                              int(bool(scores_in_workspace))))


def csa_decode(qi, w, ki, q, kc, vc, kr, vr, raw_pos0, pos0, m: int, k: int, W: int,
               scale: float, act="relu", qi_scale=None, ki_scale=None, zk=None, zv=None,
               scores=None, idx=None, out=None, lse=None, want_lse=True, ws=None,
               keep_scores=True, stream=None):
    """One whole decode step: indexer scores, top-k and attention (and, with
    zk / zv, the block the query token completes compressed into kc / vc
    first).  Returns (scores or None, idx, out, lse)."""
    return _decode(False, qi, w, ki, q, kc, vc, kr, vr, raw_pos0, pos0, m, k, W, scale, act,
                   qi_scale, ki_scale, zk, zv, scores, idx, out, lse, want_lse, ws, keep_scores,
                   stream)


def csa_decode_noalloc_max_bytes() -> int:
    return int(_lib.csa_decode_noalloc_max_bytes())


def csa_decode_noalloc(qi, w, ki, q, kc, vc, kr, vr, raw_pos0, pos0, m: int, k: int, W: int,
                       scale: float, act="relu", qi_scale=None, ki_scale=None, zk=None,
                       zv=None, scores=None, idx=None, out=None, lse=None, want_lse=True,
                       keep_scores=False, stream=None):
    """csa_decode on the library's fixed per-GPU scratch instead of a
    workspace.  The library call allocates nothing; this wrapper allocates
    only the outputs that are not passed in."""
    return _decode(True, qi, w, ki, q, kc, vc, kr, vr, raw_pos0, pos0, m, k, W, scale, act,
                   qi_scale, ki_scale, zk, zv, scores, idx, out, lse, want_lse, None,
                   keep_scores, stream)


def _decode(noalloc, qi, w, ki, q, kc, vc, kr, vr, raw_pos0, pos0, m, k, W, scale, act,
            qi_scale, ki_scale, zk, zv, scores, idx, out, lse, want_lse, ws, keep_scores,
            stream):
    dev = _dev(qi, w, ki, q, kc, pos0)
    B, T, H_I, d_I, n_cap = _index_shapes(qi, w, ki, pos0)
    Bq, Tq, H, d, n_cap2, R = _attend_shapes(q, kc, vc, kr, vr, raw_pos0, pos0, W)
    if (Bq, Tq, n_cap2) != (B, T, n_cap):
        raise ValueError("indexer and attention inputs disagree on B, T or n_cap")
    for name, t in (("zk", zk), ("zv", zv)):
        if t is not None:
            _contig(name, t)
            if t.shape != kr.shape or t.dtype != torch.float32:
                raise ValueError(f"{name} must be float32 [B, R, d]")
    if scores is None and keep_scores:
        scores = torch.empty((B, T, n_cap), dtype=torch.float32, device=dev)
    if idx is None:
        idx = torch.empty((B, T, k), dtype=torch.int32, device=dev)
    out, lse = _outputs(out, lse, B, T, H, d, dev, want_lse)
    args = (_ptr(qi), _dtype_code(qi), _ptr(qi_scale), _ptr(w), _ptr(ki), _dtype_code(ki),
            _ptr(ki_scale), _ptr(q), _ptr(kc), _ptr(vc), _dtype_code(kc), _ptr(kr), _ptr(vr),
            _ptr(zk), _ptr(zv), _ptr(raw_pos0), R, _ptr(pos0), B, T, H_I, d_I, H, d, n_cap,
            int(m), _act_code(act), int(k), int(W), float(scale), _ptr(scores), _ptr(idx),
            _ptr(out), _ptr(lse))
    if noalloc:
        _check("csa_decode_noalloc", _lib.csa_decode_noalloc(*args, _stream(stream, dev)))
    else:
        ws, nbytes = _workspace(
            ws, csa_decode_workspace_size(B, T, H, d, n_cap, k, W, scores is None), dev)
        _check("csa_decode", _lib.csa_decode(*args, _ptr(ws), nbytes, _stream(stream, dev)))
    return scores, idx, out, lse


def _bwd_common(q, kc, vc, kr, vr, raw_pos0, pos0, W, out, lse, dout):
    dev = _dev(q, kc, vc, pos0)
    B, T, H, d, n_cap, R = _attend_shapes(q, kc, vc, kr, vr, raw_pos0, pos0, W)
    for name, t, shape in (("out", out, (B, T, H, d)), ("lse", lse, (B, T, H)),
                           ("dout", dout, (B, T, H, d))):
        if t.shape != shape or t.dtype != torch.float32:
            raise ValueError(f"{name} must be float32 {list(shape)}")
        _contig(name, t)
    f32 = lambda *shape: torch.empty(shape, dtype=torch.float32, device=dev)
    grads = {"dq": f32(B, T, H, d), "dkc": f32(B, n_cap, d), "dvc": f32(B, n_cap, d),
             "dkr": f32(B, R, d) if R else None, "dvr": f32(B, R, d) if R else None}
    return dev, B, T, H, d, n_cap, R, grads


def csa_attend_backward_workspace_size(B: int, T: int, d: int, n_cap: int, k: int, W: int) -> int:
    return int(_lib.csa_attend_backward_workspace_size(B, T, d, n_cap, k, W))


def hca_attend_backward_workspace_size(B: int, T: int, d: int, n_cap: int, W: int) -> int:
    return int(_lib.hca_attend_backward_workspace_size(B, T, d, n_cap, W))


def csa_attend_backward(q, kc, vc, idx, kr, vr, raw_pos0, pos0, W: int, scale: float, out, lse,
                        dout, ws=None, stream=None) -> dict:
    """Gradients of csa_attend: returns dict dq, dkc, dvc, dkr, dvr (fp32);
    out / lse are the forward's outputs, dout the upstream gradient."""
    dev, B, T, H, d, n_cap, R, gr = _bwd_common(q, kc, vc, kr, vr, raw_pos0, pos0, W, out, lse,
                                                dout)
    if idx.dim() != 3 or idx.shape[:2] != (B, T) or idx.dtype != torch.int32:
        raise ValueError("idx must be int32 [B, T, k]")
    _contig("idx", idx)
    k = idx.shape[2]
    need = csa_attend_backward_workspace_size(B, T, d, n_cap, k, int(W))
    ws, nbytes = _workspace(ws, need, dev)
    _check("csa_attend_backward", _lib.csa_attend_backward(
        _ptr(q), _dtype_code(q), _ptr(kc), _ptr(vc), _dtype_code(kc), _ptr(idx), k, _ptr(kr),
        _ptr(vr), _ptr(raw_pos0), R, _ptr(pos0), B, T, H, d, n_cap, int(W), float(scale),
        _ptr(out), _ptr(lse), _ptr(dout), _ptr(gr["dq"]), _ptr(gr["dkc"]), _ptr(gr["dvc"]),
        _ptr(gr["dkr"]), _ptr(gr["dvr"]), _ptr(ws), nbytes, _stream(stream, dev)))
    return gr


def hca_attend_backward(q, kc, vc, m: int, kr, vr, raw_pos0, pos0, W: int, scale: float, out, lse,
                        dout, ws=None, stream=None) -> dict:
    """Gradients of hca_attend (dict as csa_attend_backward)."""
    dev, B, T, H, d, n_cap, R, gr = _bwd_common(q, kc, vc, kr, vr, raw_pos0, pos0, W, out, lse,
                                                dout)
    need = hca_attend_backward_workspace_size(B, T, d, n_cap, int(W))
    ws, nbytes = _workspace(ws, need, dev)
    _check("hca_attend_backward", _lib.hca_attend_backward(
        _ptr(q), _dtype_code(q), _ptr(kc), _ptr(vc), _dtype_code(kc), int(m), _ptr(kr), _ptr(vr),
        _ptr(raw_pos0), R, _ptr(pos0), B, T, H, d, n_cap, int(W), float(scale), _ptr(out),
        _ptr(lse), _ptr(dout), _ptr(gr["dq"]), _ptr(gr["dkc"]), _ptr(gr["dvc"]), _ptr(gr["dkr"]),
        _ptr(gr["dvr"]), _ptr(ws), nbytes, _stream(stream, dev)))
    return gr


def csa_compress_backward(x: torch.Tensor, logits: torch.Tensor, dc: torch.Tensor, m: int,
                          stream=None):
    """Gradients of csa_compress with respect to x and logits, for dc
    [B, n_tok/m, d] fp32.  Returns (dx, dlogits), fp32 [B, n_tok, d]."""
    dev = _dev(x, logits, dc)
    B, n_tok, d = x.shape
    for name, t in (("x", x), ("logits", logits)):
        if t.shape != (B, n_tok, d) or t.stride(2) != 1 or (n_tok > 1 and t.stride(1) != d):
            raise ValueError(f"{name} must be [B, n_tok, d] with contiguous rows")
    if logits.dtype != torch.float32 or dc.dtype != torch.float32:
        raise TypeError("logits and dc must be float32")
    if n_tok % m or dc.shape != (B, n_tok // m, d):
        raise ValueError("dc must be [B, n_tok / m, d] and n_tok a multiple of m")
    _contig("dc", dc)
    dx = torch.empty((B, n_tok, d), dtype=torch.float32, device=dev)
    dz = torch.empty((B, n_tok, d), dtype=torch.float32, device=dev)
    _check("csa_compress_backward", _lib.csa_compress_backward(
        _ptr(x), _dtype_code(x), _ptr(logits), _ptr(dc), B, n_tok, d, int(m), x.stride(0),
        logits.stride(0), _ptr(dx), _ptr(dz), _stream(stream, dev)))
    return dx, dz


__all__ = [
    "CSAError", "LIB_PATH", "abi_version", "last_error", "header_functions", "workspace",
    "csa_workspace_clear",
    "csa_compress", "csa_quantize_fp8_rows", "csa_quantize_mxfp4_rows", "csa_index_scores",
    "csa_topk",
    "csa_topk_workspace_size", "csa_index_topk", "csa_index_topk_workspace_size",
    "csa_decode_index_topk", "csa_select_attend", "csa_decode", "csa_decode_workspace_size",
    "csa_decode_noalloc",
    "csa_decode_noalloc_max_bytes",
    "csa_attend", "csa_attend_workspace_size", "hca_attend", "hca_attend_workspace_size",
    "csa_attend_backward", "hca_attend_backward", "csa_compress_backward",
    "csa_attend_backward_workspace_size", "hca_attend_backward_workspace_size",
]
