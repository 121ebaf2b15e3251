"""Helpers shared by the GPU parity tests (not a test module)."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

DEV = torch.device("cuda:0")


def say(*a):
    """Print and flush, so the case being run is named before GPU work."""
    print(*a, flush=True)
    sys.stdout.flush()


def decode(arr: np.ndarray) -> np.ndarray:
    """float64 values of a storage-form array (float32 or bf16 codes)."""
    if arr.dtype == np.uint16:
        return oracle.bf16_decode(arr)
    return np.asarray(arr, dtype=np.float64)


def bf16_codes(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def to_dev(arr: np.ndarray) -> torch.Tensor:
    arr = np.ascontiguousarray(arr)
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(arr).to(DEV)


def from_dev(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype in (torch.float4_e2m1fn_x2, torch.float8_e8m0fnu, torch.float8_e4m3fn):
        return t.view(torch.uint8).cpu().numpy()
    return t.cpu().numpy()


def score_close(gpu_row: np.ndarray, ref_row: np.ndarray, rel: float = 1e-3):
    """Indexer score tolerance: |d| <= rel * max(|ref|, rms(ref row)).
    Returns the worst ratio |d| / (rel * bound)."""
    if ref_row.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref_row ** 2)))
    bound = rel * np.maximum(np.abs(ref_row), max(rms, 1e-30))
    return float(np.max(np.abs(gpu_row - ref_row) / bound))


def rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def compress_bound(ref: np.ndarray, x_blocks: np.ndarray, m: int) -> np.ndarray:
    """Allowed |gpu - exact| for a compressed entry stored as bf16: half an
    ulp of bf16 rounding (taken as a full ulp for margin) plus the fp32
    accumulation error of an m-term weighted sum, which is relative to the
    block's largest |x| rather than to the (possibly cancelling) result.
    x_blocks: [n_blocks, m, d]."""
    a = np.maximum(np.abs(ref), 2.0 ** -126)
    ulp = 2.0 ** (np.floor(np.log2(a)) - 7)
    return ulp + m * 2.0 ** -22 * np.abs(x_blocks).max(axis=1)
