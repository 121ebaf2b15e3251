"""The seeded workloads have the shapes of the five configurations the hot
path is measured on (transcribed here from their statements), so a change
to workloads/ that silently shrinks a benchmark fails on the CPU.

  tiny prefill: 1 x 2048 tokens, fp32, d 64, m 4 -> 512 entries, indexer
    4 x 64, top-64, 8 heads, window 32
  128K decode: batch 32, 131072 context tokens -> 32768 entries at m 4, d
    128, indexer 64 x 128, top-1024, 64 heads, window 128, 16 planted
  chunked prefill: 8192 new tokens after 262144 (65536 + 2048 entries),
    indexer 64 x 128, top-1024, 64 heads, window 128
  HCA 1M: batch 16, 1048576 tokens at m' 128 -> 8192 entries, 64 heads,
    window 128, no indexer
  1M fp8 decode: batch 4, 1048576 tokens -> 262144 entries at m 4, fp8
    indexer keys with a scale per entry, top-1024, 64 planted, evenly spread
"""

import workloads as WL


def test_tiny_prefill():
    c = WL.TINY_PREFILL_F32
    assert (c.B, c.T, c.pos0, c.storage, c.d, c.m) == (1, 2048, 0, "f32", 64, 4)
    assert c.n_cap == 512 and (c.H_I, c.d_I, c.k, c.H, c.W) == (4, 64, 64, 8, 32)


def test_decode_128k():
    c = WL.DECODE_128K_BF16
    assert (c.B, c.T, c.pos0, c.storage, c.d, c.m) == (32, 1, 131072, "bf16", 128, 4)
    assert c.n_cap == 32768 and (c.pos0 + 1) // c.m == 32768
    assert (c.H_I, c.d_I, c.k, c.H, c.W, c.planted) == (64, 128, 1024, 64, 128, 16)


def test_chunked_prefill():
    c = WL.PREFILL_256K_BF16
    assert (c.B, c.T, c.pos0, c.n_new_tokens, c.storage) == (1, 8192, 262144, 8192, "bf16")
    assert (c.n_ctx_entries, c.n_cap) == (65536, 65536 + 2048)
    assert (c.H_I, c.d_I, c.k, c.H, c.d, c.W) == (64, 128, 1024, 64, 128, 128)


def test_hca_1m():
    c = WL.HCA_DECODE_1M_BF16
    assert (c.B, c.T, c.pos0, c.m, c.storage) == (16, 1, 1048576, 128, "bf16")
    assert c.n_cap == 8192 and c.hca and c.k == 0
    assert (c.H, c.d, c.W) == (64, 128, 128)


def test_decode_1m_fp8():
    c = WL.DECODE_1M_FP8
    assert (c.B, c.T, c.pos0, c.m, c.storage, c.ki_fp8) == (4, 1, 1048576, 4, "bf16", True)
    assert c.n_cap == 262144
    assert (c.H_I, c.d_I, c.k, c.H, c.d, c.W) == (64, 128, 1024, 64, 128, 128)
    assert c.planted == 64 and c.planted_spread
