"""fp64 reference for attention over a paged KV cache -- TEST INFRASTRUCTURE ONLY.

Page "why FA is 2x on A100 but 1.5x on Ascend 910" (section 5) recommends
managing the inference KV cache with PagedAttention: the keys and values of a
sequence live in fixed-size pages of a shared pool, and a per-sequence page
table lists which pages hold it.  The pages give no further detail; the
plainest reading (the one this oracle follows) is:

  cache (num_pages, page_size, Hkv, D); key j of sequence s is row
  j % page_size of page block_table[s, j // page_size], for j < seqlens_k[s].

The attention itself is the standard definition of attention.py: the new
queries of sequence s (rows cu_seqlens_q[s]:cu_seqlens_q[s+1] of q) attend to
that sequence's seqlens_k[s] keys, causal with bottom-right alignment (query i
of Lq sees keys j <= i + Lk - Lq: new tokens sit at the end of the cache).
The oracle gathers each sequence's keys and values from the pages into
contiguous arrays (no tiling, no split) and calls attention_one.

attention_paged_fp8kv is the same attention over a cache stored as 8-bit
floats (the same page, section 5, recommends a narrower KV cache to halve the
bytes moved): the pages hold OCP E4M3 bytes (decoded by fp8.e4m3_to_f64) and
one float factor per tensor; q stays bf16.
"""

from __future__ import annotations

import numpy as np

from .attention import attention_one, bf16_bits_to_f64
from .fp8 import e4m3_to_f64


def gather_pages(cache, block_table_row, seqlen: int):
    """The first `seqlen` logical rows of one sequence, (seqlen, Hkv, D)."""
    page_size = cache.shape[1]
    j = np.arange(seqlen)
    pages = np.asarray(block_table_row, dtype=np.int64)[j // page_size]
    return cache[pages, j % page_size]


def attention_paged(q_bits, k_cache_bits, v_cache_bits, cu_seqlens_q, seqlens_k, block_table,
                    scale, causal: bool):
    """q (Tq, Hq, D) bf16 bits; k/v caches (num_pages, page_size, Hkv, D) bf16
    bits; block_table (num_seqs, max_pages) int; seqlens_k (num_seqs,).
    Returns O (Tq, Hq, D) float64 and LSE (Hq, Tq) float64."""
    q = bf16_bits_to_f64(q_bits)
    tq, hq, d = q.shape
    hkv = k_cache_bits.shape[2]
    group = hq // hkv
    o = np.zeros((tq, hq, d))
    lse = np.full((hq, tq), -np.inf)
    cq = np.asarray(cu_seqlens_q, dtype=np.int64)
    for s in range(len(cq) - 1):
        q0, q1 = cq[s], cq[s + 1]
        if q1 == q0:
            continue
        lk = int(seqlens_k[s])
        k = bf16_bits_to_f64(gather_pages(k_cache_bits, block_table[s], lk))
        v = bf16_bits_to_f64(gather_pages(v_cache_bits, block_table[s], lk))
        for h in range(hq):
            g = h // group
            o[q0:q1, h], lse[h, q0:q1] = attention_one(q[q0:q1, h], k[:, g], v[:, g],
                                                       np.float32(scale), causal)
    return o, lse


def attention_paged_fp8kv(q_bits, k_cache8, v_cache8, cu_seqlens_q, seqlens_k, block_table,
                          scale, k_scale, v_scale, causal: bool):
    """As attention_paged with E4M3 cache pages (bytes) and per-tensor factors."""
    q = bf16_bits_to_f64(q_bits)
    tq, hq, d = q.shape
    hkv = k_cache8.shape[2]
    group = hq // hkv
    ks = float(np.float32(k_scale))
    vs = float(np.float32(v_scale))
    o = np.zeros((tq, hq, d))
    lse = np.full((hq, tq), -np.inf)
    cq = np.asarray(cu_seqlens_q, dtype=np.int64)
    for s in range(len(cq) - 1):
        q0, q1 = cq[s], cq[s + 1]
        if q1 == q0:
            continue
        lk = int(seqlens_k[s])
        k = e4m3_to_f64(gather_pages(k_cache8, block_table[s], lk)) * ks
        v = e4m3_to_f64(gather_pages(v_cache8, block_table[s], lk)) * vs
        for h in range(hq):
            g = h // group
            o[q0:q1, h], lse[h, q0:q1] = attention_one(q[q0:q1, h], k[:, g], v[:, g],
                                                       np.float32(scale), causal)
    return o, lse
