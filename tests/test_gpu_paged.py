"""GPU parity of attention over a paged KV cache (attn_fwd_paged) against the
fp64 oracle (oracle.attention_paged).

Covers decode (one query per sequence), speculative decode (a few queries,
causal), chunked prefill (several 32-row blocks), Lq > Lk, empty sequences,
page sizes 16..256 including a non-power of two, GQA groups 1..8, NaN in every
cache row no sequence owns, forced key-range splits, the dense-cache layout,
out-of-pool page numbers, and a full-size decode batch checked on sampled
sequences.
"""

from __future__ import annotations

import os

import numpy as np
import pytest

import oracle
from synth import gen
from tests.gpu_util import check_lse, check_o, dev_bf16, dev_i32, host

pytestmark = pytest.mark.gpu


def api():
    import tiled_attention_fwd_amd as t
    return t


def run(w, workspace=False, table=None):
    t = api()
    ws = None
    if workspace:
        ws = t.paged_workspace(len(w.lengths_q), w.max_seqlen_q, max(w.max_seqlen_k, 1), w.hq,
                               w.hkv, w.d)
    o, lse = t.attn_fwd_paged(dev_bf16(w.q), dev_bf16(w.k_cache), dev_bf16(w.v_cache),
                              dev_i32(w.cu_seqlens_q), dev_i32(w.seqlens_k),
                              dev_i32(w.block_table if table is None else table),
                              max(w.max_seqlen_q, 1), w.max_seqlen_k, scale=float(w.scale),
                              causal=w.causal, workspace=ws)
    return host(o), host(lse)


def ref(w):
    return oracle.attention_paged(w.q, w.k_cache, w.v_cache, w.cu_seqlens_q, w.seqlens_k,
                                  w.block_table, w.scale, w.causal)


def check(w, **kw):
    o, lse = run(w, **kw)
    o_ref, lse_ref = ref(w)
    return check_o(o, o_ref), check_lse(lse, lse_ref)


@pytest.mark.parametrize("d", [32, 64, 128, 256])
@pytest.mark.parametrize("page", [16, 48, 64])
def test_decode_gqa_ragged(d, page):
    w = gen.make_paged(f"dec{d}_{page}", 1000 + d + page, [1] * 6, [1, 17, 300, 1000, 64, 33],
                       8, 2, d, page, True, fill=float("nan"))
    print(check(w))


@pytest.mark.parametrize("group", [1, 4, 8])
def test_speculative_decode_causal(group):
    hkv = 2
    w = gen.make_paged(f"spec{group}", 1100 + group, [4, 2, 3, 1], [100, 33, 257, 4], group * hkv,
                       hkv, 128, 32, True, fill=float("nan"))
    print(check(w))


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("d", [32, 64, 256])
def test_chunked_prefill_several_row_blocks(causal, d):
    w = gen.make_paged("chunk", 1200 + d, [70, 5, 0, 33], [200, 40, 9, 33], 8, 2, d, 16, causal,
                       fill=float("nan"))
    print(check(w))


def test_lq_gt_lk_and_empty():
    w = gen.make_paged("qgk", 1300, [6, 3, 0, 2], [3, 0, 5, 40], 4, 4, 128, 16, True,
                       fill=float("nan"))
    o, lse = run(w)
    o_ref, lse_ref = ref(w)
    check_o(o, o_ref)
    check_lse(lse, lse_ref)
    # queries that see no key: exactly 0 and -inf
    assert np.all(o[:3] == 0.0) and np.all(lse[:, :3] == -np.inf)
    assert np.all(o[6:9] == 0.0)


@pytest.mark.parametrize("chunk", ["1", "3"])
@pytest.mark.parametrize("d", [32, 64, 128, 256])
def test_forced_split_matches_oracle(monkeypatch, chunk, d):
    monkeypatch.setenv("ATTN_PAGED_CHUNK_TILES", chunk)
    w = gen.make_paged(f"split{chunk}", 1400 + d, [1, 3, 2, 1], [500, 70, 0, 31], 8, 2, d, 32,
                       True, fill=float("nan"))
    assert api().attn_fwd_paged_workspace_bytes(4, w.max_seqlen_q, w.max_seqlen_k, 8, 2, d) > 0
    print(check(w, workspace=True))


def test_auto_split_decode():
    # few workgroups and long key ranges: the planner splits by itself
    w = gen.make_paged("auto", 1500, [1, 1], [4000, 2500], 8, 1, 128, 64, True)
    assert api().attn_fwd_paged_workspace_bytes(2, 1, 4000, 8, 1, 128) > 0
    a = check(w, workspace=True)
    b = check(w, workspace=False)
    print(a, b)


def test_dense_cache_layout():
    # (B, Lmax, Hkv, D) cache: page_size = Lmax, block_table[s] = s
    r = np.random.Generator(np.random.PCG64(16))
    b, lmax, hq, hkv, d = 3, 256, 8, 2, 128
    lens_k = [256, 100, 7]
    w = gen.make_paged("dense", 1600, [2, 1, 1], lens_k, hq, hkv, d, 256, True, spare_pages=0)
    w.k_cache = gen.normal_bf16(r, (b, lmax, hkv, d))
    w.v_cache = gen.normal_bf16(r, (b, lmax, hkv, d))
    w.block_table = np.arange(b, dtype=np.int32).reshape(b, 1)
    print(check(w))


def test_out_of_pool_page_reads_zero_keys():
    w = gen.make_paged("oop", 1700, [1, 2], [40, 50], 4, 2, 64, 16, False)
    n = w.k_cache.shape[0]
    bad = w.block_table.copy()
    bad[0, 1] = n + 5          # keys 16..31 of sequence 0 name a page outside the pool
    o, lse = run(w, table=bad)
    # expected: the same table pointing at an all-zero page appended to the pool
    zk = np.concatenate([w.k_cache, np.zeros_like(w.k_cache[:1])])
    zv = np.concatenate([w.v_cache, np.zeros_like(w.v_cache[:1])])
    good = w.block_table.copy()
    good[0, 1] = n
    o_ref, lse_ref = oracle.attention_paged(w.q, zk, zv, w.cu_seqlens_q, w.seqlens_k, good,
                                            w.scale, False)
    check_o(o, o_ref)
    check_lse(lse, lse_ref)


def test_full_size_decode_batch_sampled():
    """32 sequences, 64 query heads over 8 KV heads, d=128, one new token each,
    4096..8192 cached keys in 64-key pages; the oracle checks 4 sequences."""
    r = np.random.Generator(np.random.PCG64(1800))
    lens = [int(x) for x in r.integers(4096, 8193, size=32)]
    w = gen.make_paged("decode_b32", 1801, [1] * 32, lens, 64, 8, 128, 64, True)
    t = api()
    ws = t.paged_workspace(32, 1, max(lens), 64, 8, 128)
    o, lse = t.attn_fwd_paged(dev_bf16(w.q), dev_bf16(w.k_cache), dev_bf16(w.v_cache),
                              dev_i32(w.cu_seqlens_q), dev_i32(w.seqlens_k),
                              dev_i32(w.block_table), 1, max(lens), scale=float(w.scale),
                              causal=True, workspace=ws)
    o, lse = host(o), host(lse)
    for s in (0, 7, 19, 31):
        sub = gen.make_paged("x", 1, [1], [1], 64, 8, 128, 64, True)  # container, fields replaced
        sub.q = w.q[s:s + 1]
        sub.k_cache, sub.v_cache = w.k_cache, w.v_cache
        sub.block_table = w.block_table[s:s + 1]
        sub.seqlens_k = w.seqlens_k[s:s + 1]
        sub.cu_seqlens_q = np.array([0, 1], dtype=np.int32)
        o_ref, lse_ref = ref(sub)
        check_o(o[s:s + 1], o_ref, f"seq {s}")
        check_lse(lse[:, s:s + 1], lse_ref, f"seq {s}")


@pytest.mark.parametrize("page", [16, 32])
def test_many_short_decode_sequences_two_workgroups_per_cu(page):
    """72 sequences x 8 KV heads at d=64 (576 workgroups, no split): the
    default layout of four waves of two stages, two workgroups per CU; ragged
    key lengths from 1 to 700 and NaN in every cache row no sequence owns."""
    r = np.random.Generator(np.random.PCG64(1900 + page))
    lens = [int(x) for x in r.integers(1, 701, size=72)]
    w = gen.make_paged(f"many{page}", 1901 + page, [1] * 72, lens, 8, 8, 64, page, True,
                       fill=float("nan"))
    t = api()
    plan_ws = t.attn_fwd_paged_workspace_bytes(72, 1, max(lens), 8, 8, 64)
    assert plan_ws == 0  # no split: 576 workgroups already
    print(check(w))


@pytest.mark.parametrize("d,lk", [(128, 6000), (64, 9500), (32, 7000), (256, 3000)])
def test_long_sequence_without_split(d, lk):
    # no workspace: one workgroup walks the whole key range, more than 32 tiles
    # per wave (the page numbers are fetched in batches of 32 tiles)
    w = gen.make_paged(f"long{d}", 1900 + d, [1, 2], [lk, 700], 8, 2, d, 16, True,
                       fill=float("nan"))
    print(check(w, workspace=False))


# ---------------------------------------------------------------- E4M3 cache
def run_f8(w, k8, v8, kf, vf, workspace):
    import torch
    t = api()
    u8 = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda")
    ws = None
    if workspace:
        ws = t.paged_workspace(len(w.lengths_q), max(w.max_seqlen_q, 1), max(w.max_seqlen_k, 1),
                               w.hq, w.hkv, w.d)
    o, lse = t.attn_fwd_paged_fp8kv(dev_bf16(w.q), u8(k8), u8(v8), dev_i32(w.cu_seqlens_q),
                                    dev_i32(w.seqlens_k), dev_i32(w.block_table),
                                    max(w.max_seqlen_q, 1), w.max_seqlen_k, scale=float(w.scale),
                                    k_scale=kf, v_scale=vf, causal=w.causal, workspace=ws)
    return host(o), host(lse)


def _climbing_cache(w, cache, code):
    """Every head and dim of each sequence's key rows set to code(p) for 2^p,
    p rising from -4 to 4 along the sequence."""
    out = cache.copy()
    for s, lk in enumerate(w.seqlens_k):
        lk = int(lk)
        p = np.floor(-4 + 8 * np.arange(lk) / max(lk - 1, 1)).astype(np.int64)
        for j in range(lk):
            out[w.block_table[s, j // w.page_size], j % w.page_size] = code(int(p[j]))
    return out


@pytest.mark.parametrize("d", [64, 128])
def test_decode_row_maximum_climbing(d):
    """Q = 1 and cached keys 2^-4 .. 2^4 rising along each sequence: the row
    maxima climb past the 2^8 lazy-rescale threshold many times (bf16 cache
    with and without a split, E4M3 cache)."""
    w = gen.make_paged("dclimb", 1500 + d, [1, 4, 1], [1000, 300, 64], 8, 2, d, 16, True,
                       fill=float("nan"))
    bf = lambda x: gen.bf16_bits_from_f32(np.array([x], dtype=np.float32))[0]
    w.q = np.full_like(w.q, bf(1.0))
    w.k_cache = _climbing_cache(w, w.k_cache, lambda p: bf(2.0 ** p))
    print(check(w), check(w, workspace=True))
    k8, v8 = gen.paged_cache_e4m3(w, 1500 + d)
    k8 = _climbing_cache(w, k8, lambda p: np.uint8((p + 7) << 3))  # E4M3 2^p
    o, lse = run_f8(w, k8, v8, 1.0, 1.0, False)
    o_ref, lse_ref = oracle.attention_paged_fp8kv(w.q, k8, v8, w.cu_seqlens_q, w.seqlens_k,
                                                  w.block_table, w.scale, 1.0, 1.0, True)
    print(check_o(o, o_ref), check_lse(lse, lse_ref))


@pytest.mark.parametrize("d", [32, 64, 128, 256])
@pytest.mark.parametrize("page,workspace", [(16, False), (64, True), (48, True)])
def test_fp8_cache_decode_and_spec(d, page, workspace):
    w = gen.make_paged(f"f8c{d}", 2500 + d + page, [1, 4, 2, 1, 0], [7, 300, 1000, 64, 5], 8, 2,
                       d, page, True, fill=float("nan"))
    for kf, vf in ((1.0, 1.0), (0.5, 2.0)):
        k8, v8 = gen.paged_cache_e4m3(w, 2500 + d, (kf, vf))
        o, lse = run_f8(w, k8, v8, kf, vf, workspace)
        o_ref, lse_ref = oracle.attention_paged_fp8kv(w.q, k8, v8, w.cu_seqlens_q, w.seqlens_k,
                                                      w.block_table, w.scale, kf, vf, True)
        print(check_o(o, o_ref), check_lse(lse, lse_ref))


@pytest.mark.parametrize("d", [32, 128, 256])
def test_fp8_cache_chunked_prefill_noncausal(d):
    w = gen.make_paged("f8cp", 2600 + d, [70, 5], [200, 40], 8, 2, d, 32, False, fill=float("nan"))
    k8, v8 = gen.paged_cache_e4m3(w, 2600 + d)
    o, lse = run_f8(w, k8, v8, 1.0, 1.0, False)
    o_ref, lse_ref = oracle.attention_paged_fp8kv(w.q, k8, v8, w.cu_seqlens_q, w.seqlens_k,
                                                  w.block_table, w.scale, 1.0, 1.0, False)
    print(check_o(o, o_ref), check_lse(lse, lse_ref))
