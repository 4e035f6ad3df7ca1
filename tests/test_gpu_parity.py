"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Sizes span several query and key tiles and leave ragged tails.  Every case
uses seeded synthetic inputs from synth/; expected values come only from
oracle/.
"""

from __future__ import annotations

import math
import os

import numpy as np
import pytest

import oracle
from synth import gen
from tests.gpu_util import check_lse, check_o, dev_bf16, dev_i32, host

pytestmark = pytest.mark.gpu

D_ALL = [32, 64, 128, 256]


def api():
    import tiled_attention_fwd_amd as t
    return t


def run_varlen(w, causal=None, return_lse=True):
    t = api()
    causal = w.causal if causal is None else causal
    o, lse = t.attn_fwd_varlen(dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v),
                               dev_i32(w.cu_seqlens_q), dev_i32(w.cu_seqlens_k), w.max_seqlen,
                               scale=float(w.scale), causal=causal, return_lse=return_lse)
    return host(o), (host(lse) if lse is not None else None)


def run_dense(w, return_lse=True):
    t = api()
    o, lse = t.attn_fwd_dense(dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v), scale=float(w.scale),
                              causal=w.causal, return_lse=return_lse)
    return host(o), (host(lse) if lse is not None else None)


# ----------------------------------------------------------------------------- varlen
@pytest.mark.parametrize("d", D_ALL)
@pytest.mark.parametrize("causal", [True, False])
def test_varlen_ragged_gqa(d, causal):
    lens = [1, 7, 64, 100, 129, 300, 33]
    w = gen.make_varlen(f"vr{d}", 100 + d, lens, 4, 2, d, causal)
    o, lse = run_varlen(w)
    o_ref, lse_ref = oracle.attention_varlen(w.q, w.k, w.v, w.cu_seqlens_q, w.cu_seqlens_k,
                                             w.scale, causal)
    print(d, causal, check_o(o, o_ref), check_lse(lse, lse_ref))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_varlen_lq_ne_lk_and_empty_sequences(d, causal):
    lq = [5, 130, 0, 64, 3, 0]
    lk = [9, 70, 12, 200, 0, 0]
    w = gen.make_varlen("ne", 200 + d, lq, 2, 2, d, causal, lengths_k=lk)
    o, lse = run_varlen(w)
    o_ref, lse_ref = oracle.attention_varlen(w.q, w.k, w.v, w.cu_seqlens_q, w.cu_seqlens_k,
                                             w.scale, causal)
    print(check_o(o, o_ref), check_lse(lse, lse_ref))


def test_varlen_without_lse():
    w = gen.make_varlen("nolse", 301, [70, 5], 2, 1, 128, True)
    o, lse = run_varlen(w, return_lse=False)
    assert lse is None
    o_ref, _ = oracle.attention_varlen(w.q, w.k, w.v, w.cu_seqlens_q, w.cu_seqlens_k, w.scale, True)
    check_o(o, o_ref)


def test_varlen_32x64_full_size():
    w = gen.build_workload("varlen_32x64")
    o, lse = run_varlen(w)
    o_ref, lse_ref = oracle.attention_varlen(w.q, w.k, w.v, w.cu_seqlens_q, w.cu_seqlens_k,
                                             w.scale, True)
    print(check_o(o, o_ref), check_lse(lse, lse_ref))


# ----------------------------------------------------------------------------- dense
@pytest.mark.parametrize("d", D_ALL)
@pytest.mark.parametrize("causal", [True, False])
def test_dense_ragged(d, causal):
    w = gen.make_dense(f"dn{d}", 400 + d, 2, 200, 200, 3, 3, d, causal)
    o, lse = run_dense(w)
    o_ref, lse_ref = oracle.attention_dense(w.q, w.k, w.v, w.scale, causal)
    print(check_o(o, o_ref), check_lse(lse, lse_ref))


def test_dense_gqa_lq_ne_lk():
    w = gen.make_dense("dg", 501, 2, 77, 190, 8, 2, 128, True)
    o, lse = run_dense(w)
    o_ref, lse_ref = oracle.attention_dense(w.q, w.k, w.v, w.scale, True)
    print(check_o(o, o_ref), check_lse(lse, lse_ref))


def test_dense_strided_views():
    import torch
    t = api()
    w = gen.make_dense("st", 502, 2, 150, 150, 4, 4, 64, False)
    # BHSD storage viewed as BSHD: non-contiguous seq/head strides
    q = dev_bf16(np.ascontiguousarray(w.q.transpose(0, 2, 1, 3))).permute(0, 2, 1, 3)
    k = dev_bf16(np.ascontiguousarray(w.k.transpose(0, 2, 1, 3))).permute(0, 2, 1, 3)
    v = dev_bf16(np.ascontiguousarray(w.v.transpose(0, 2, 1, 3))).permute(0, 2, 1, 3)
    out = torch.empty((2, 4, 150, 64), dtype=torch.float32, device="cuda").permute(0, 2, 1, 3)
    o, lse = t.attn_fwd_dense(q, k, v, scale=float(w.scale), causal=False, out=out)
    o_ref, lse_ref = oracle.attention_dense(w.q, w.k, w.v, w.scale, False)
    check_o(host(o.contiguous()), o_ref)
    check_lse(host(lse), lse_ref)


@pytest.mark.parametrize("policy", ["18", "19", "20"])
def test_newer_dma_policies_dense_lq_ne_lk_and_strided(policy):
    # the four-key-group and 128-key-tile policies on the dense layout:
    # bottom-right causal with Lk > Lq and Lk < Lq, then BHSD storage viewed
    # as BSHD (non-contiguous strides) with a strided output
    import torch
    t = api()
    os.environ["ATTN_FWD_TILE"] = policy
    try:
        for sq, sk in ((300, 520), (520, 300)):
            w = gen.make_dense(f"nd{sq}", 1700 + sq, 2, sq, sk, 4, 2, 128, True)
            o, lse = run_dense(w)
            o_ref, lse_ref = oracle.attention_dense(w.q, w.k, w.v, w.scale, True)
            check_o(o, o_ref)
            check_lse(lse, lse_ref)
        w = gen.make_dense("ns", 1750, 2, 300, 300, 4, 4, 64, False)
        q = dev_bf16(np.ascontiguousarray(w.q.transpose(0, 2, 1, 3))).permute(0, 2, 1, 3)
        k = dev_bf16(np.ascontiguousarray(w.k.transpose(0, 2, 1, 3))).permute(0, 2, 1, 3)
        v = dev_bf16(np.ascontiguousarray(w.v.transpose(0, 2, 1, 3))).permute(0, 2, 1, 3)
        out = torch.empty((2, 4, 300, 64), dtype=torch.float32, device="cuda").permute(0, 2, 1, 3)
        o, lse = t.attn_fwd_dense(q, k, v, scale=float(w.scale), causal=False, out=out)
        o_ref, lse_ref = oracle.attention_dense(w.q, w.k, w.v, w.scale, False)
        check_o(host(o.contiguous()), o_ref)
        check_lse(host(lse), lse_ref)
    finally:
        del os.environ["ATTN_FWD_TILE"]


# ----------------------------------------------------------------------------- closed forms on GPU
@pytest.mark.parametrize("d", [64, 128])
def test_zero_query_gives_prefix_mean_and_log_count(d):
    w = gen.make_varlen("z", 600 + d, [300, 17], 2, 2, d, True)
    w.q[:] = 0
    o, lse = run_varlen(w)
    v = oracle.bf16_bits_to_f64(w.v)
    c = w.cu_seqlens_q
    for s in range(2):
        n = np.arange(1, c[s + 1] - c[s] + 1)
        np.testing.assert_allclose(lse[:, c[s]:c[s + 1]], np.log(n)[None, :].repeat(2, 0),
                                   rtol=0, atol=1e-5)
        pref = np.cumsum(v[c[s]:c[s + 1]], axis=0) / n[:, None, None]
        check_o(o[c[s]:c[s + 1]], pref)


def test_onehot_future_target_is_masked():
    # Hadamard keys: each query's dominant key is in its future; a leaking mask
    # would return that key's value row instead of the prefix mean.
    d, L = 64, 64
    h = np.array([[1.0]])
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    kbits = gen.bf16_bits_from_f32((3.0 * h[:L]).astype(np.float32))
    tgt = [min(i + 1 + (i % 5), L - 1) for i in range(L)]
    qf = 3.0 * h[tgt]
    qf[L - 1] = 0.0
    w = gen.make_varlen("oh", 700, [L], 1, 1, d, True)
    w.q[:, 0] = gen.bf16_bits_from_f32(qf.astype(np.float32))
    w.k[:, 0] = kbits
    o, lse = run_varlen(w)
    v = oracle.bf16_bits_to_f64(w.v)[:, 0]
    pref = np.cumsum(v, axis=0) / np.arange(1, L + 1)[:, None]
    check_o(o[:, 0], pref)
    np.testing.assert_allclose(lse[0], np.log(np.arange(1, L + 1)), rtol=0, atol=1e-4)


# ----------------------------------------------------------------------------- scheduling invariance
def test_sequence_alone_equals_sequence_in_pack_bitwise():
    os.environ["ATTN_FWD_TILE"] = "0"
    try:
        lens = [100, 257, 31, 512]
        w = gen.make_varlen("pk", 800, lens, 4, 4, 128, True)
        o_pack, l_pack = run_varlen(w)
        c = w.cu_seqlens_q
        for s, L in enumerate(lens):
            ws = gen.make_varlen("one", 1, [L], 4, 4, 128, True)
            ws.q[:] = w.q[c[s]:c[s + 1]]
            ws.k[:] = w.k[c[s]:c[s + 1]]
            ws.v[:] = w.v[c[s]:c[s + 1]]
            o1, l1 = run_varlen(ws)
            assert np.array_equal(o1, o_pack[c[s]:c[s + 1]])
            assert np.array_equal(l1, l_pack[:, c[s]:c[s + 1]])
            # dense path on the same sequence gives the same bits too
            wd = gen.make_dense("dd", 1, 1, L, L, 4, 4, 128, True)
            wd.q[0] = ws.q
            wd.k[0] = ws.k
            wd.v[0] = ws.v
            od, ld = run_dense(wd)
            assert np.array_equal(od[0], o1) and np.array_equal(ld[0], l1)
    finally:
        del os.environ["ATTN_FWD_TILE"]


def test_repeat_runs_are_bitwise_identical():
    w = gen.make_varlen("rep", 900, [1000, 3, 600], 8, 2, 128, True)
    a = run_varlen(w)
    b = run_varlen(w)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_future_perturbation_leaves_prefix_bitwise():
    w = gen.make_varlen("fp", 901, [400], 2, 2, 128, True)
    o1, l1 = run_varlen(w)
    w.k[250:] = gen.bf16_bits_from_f32(np.full(w.k[250:].shape, 7.0, np.float32))
    w.v[250:] = gen.bf16_bits_from_f32(np.full(w.v[250:].shape, -3.0, np.float32))
    o2, l2 = run_varlen(w)
    assert np.array_equal(o1[:250], o2[:250]) and np.array_equal(l1[:, :250], l2[:, :250])


def compiled(policy, d) -> bool:
    """Whether the library compiles tile policy `policy` for head_dim d (some
    are left out for register or LDS budget); asked of the library itself."""
    return api().attn_fwd_tile_policy_compiled(int(policy), d)


@pytest.mark.parametrize("policy", [str(i) for i in range(21)])
@pytest.mark.parametrize("causal", [True, False])
def test_every_compiled_tile_policy(policy, causal):
    os.environ["ATTN_FWD_TILE"] = policy
    try:
        for d in D_ALL:
            if not compiled(policy, d):
                continue
            w = gen.make_varlen("pol", 1000 + d, [150, 64, 1, 90, 700], 2, 1, d, causal)
            o, lse = run_varlen(w)
            o_ref, lse_ref = oracle.attention_varlen(w.q, w.k, w.v, w.cu_seqlens_q,
                                                     w.cu_seqlens_k, w.scale, causal)
            check_o(o, o_ref)
            check_lse(lse, lse_ref)
    finally:
        del os.environ["ATTN_FWD_TILE"]


def climbing_keys(k_bits, cu_k, lo=-4, hi=4):
    """K rows set to 2^p in every head and dim, p rising from lo to hi along
    each sequence (bf16 bits)."""
    k = k_bits.copy()
    for s in range(len(cu_k) - 1):
        k0, k1 = int(cu_k[s]), int(cu_k[s + 1])
        p = np.floor(lo + (hi - lo) * np.arange(k1 - k0) / max(k1 - k0 - 1, 1))
        k[k0:k1] = gen.bf16_bits_from_f32(np.exp2(p).astype(np.float32))[:, None, None]
    return k


@pytest.mark.parametrize("policy", [str(i) for i in range(21)])
def test_row_maximum_climbing_every_policy(policy):
    """Q = 1 and keys 2^-4 .. 2^4 rising along each sequence: a row's maximum
    climbs by up to ~130 binades at a time (to ~260 at head_dim 128), far past
    the 2^8 lazy-rescale threshold, so every policy's rescale branch runs after
    its first tile as well as on it."""
    os.environ["ATTN_FWD_TILE"] = policy
    try:
        one = gen.bf16_bits_from_f32(np.array([1.0], dtype=np.float32))[0]
        for d in D_ALL:
            if not compiled(policy, d):
                continue
            w = gen.make_varlen("climb", 1300 + d, [700, 150, 64], 2, 1, d, True)
            w.q = np.full_like(w.q, one)
            w.k = climbing_keys(w.k, w.cu_seqlens_k)
            o, lse = run_varlen(w)
            o_ref, lse_ref = oracle.attention_varlen(w.q, w.k, w.v, w.cu_seqlens_q,
                                                     w.cu_seqlens_k, w.scale, True)
            check_o(o, o_ref)
            check_lse(lse, lse_ref)
    finally:
        del os.environ["ATTN_FWD_TILE"]


@pytest.mark.parametrize("causal", [True, False])
def test_default_policy_one_round_of_64_query_blocks(causal):
    # head_dim 128, 512..4096 queries and at most 512 blocks of 64 queries:
    # the default is the four-key-group policy (its merge runs in two rounds)
    assert "ATTN_FWD_TILE" not in os.environ
    w = gen.make_varlen("kg4", 1210, [1024, 700], 4, 2, 128, causal)
    o, lse = run_varlen(w)
    o_ref, lse_ref = oracle.attention_varlen(w.q, w.k, w.v, w.cu_seqlens_q, w.cu_seqlens_k,
                                             w.scale, causal)
    check_o(o, o_ref)
    check_lse(lse, lse_ref)


@pytest.mark.parametrize("hq,hkv", [(8, 2), (12, 4)])
def test_multi_sequence_block_orders_varlen(hq, hkv):
    # several sequences on the DMA-staged kernel: sequence-major order when
    # hq % 8 == 0, unit-major order otherwise
    assert "ATTN_FWD_TILE" not in os.environ
    w = gen.make_varlen(f"ord{hq}", 1300 + hq, [700, 300, 1100], hq, hkv, 128, True)
    o, lse = run_varlen(w)
    o_ref, lse_ref = oracle.attention_varlen(w.q, w.k, w.v, w.cu_seqlens_q, w.cu_seqlens_k,
                                             w.scale, True)
    check_o(o, o_ref)
    check_lse(lse, lse_ref)


def test_multi_sequence_block_order_pipelined_dense_batch():
    # a batch on the software-pipelined kernel (policy 14, head_dim 64,
    # non-causal): unit-major order, with a grid padded to whole rounds of 8 units
    os.environ["ATTN_FWD_TILE"] = "14"
    try:
        w = gen.make_dense("ordp", 1320, 6, 1024, 1024, 12, 12, 64, False)
        o, lse = run_dense(w)
    finally:
        os.environ.pop("ATTN_FWD_TILE", None)
    o_ref, lse_ref = oracle.attention_dense(w.q, w.k, w.v, w.scale, False)
    check_o(o, o_ref)
    check_lse(lse, lse_ref)


# Shapes that reach each branch of the default tile selection (head_dim,
# causal, number of workgroups per block size), run with a split workspace as
# a caller that passes one would: (name, head_dim, causal, lengths, heads q/kv,
# policy the selection picks).
DEFAULT_BRANCHES = [
    ("d32_c_few", 32, True, [300, 290], 4, 2, "20"),
    ("d32_c_many", 32, True, [256] * 64, 16, 4, "19"),
    ("d32_n_many", 32, False, [256] * 16, 16, 16, "19"),
    ("d64_c_many", 64, True, [256] * 80, 8, 2, "13"),
    ("d64_c_kg4", 64, True, [1024, 900], 8, 2, "18"),
    ("d64_c_kg2", 64, True, [2048, 1500], 16, 4, "12"),
    ("d64_n_kg4", 64, False, [1024], 4, 2, "18"),
    ("d64_n_kg2", 64, False, [1024, 1000], 16, 4, "12"),
    ("d64_n_few", 64, False, [300, 290], 4, 2, "20"),
    ("d64_n_mid", 64, False, [256] * 16, 16, 4, "19"),
    ("d64_n_many", 64, False, [256] * 32, 16, 4, "13"),
    ("d128_n_round", 128, False, [256] * 16, 16, 4, "19"),
    ("d128_n_kg4", 128, False, [600], 4, 2, "18"),
    ("d128_n_split", 128, False, [1024] * 4, 8, 2, "12"),
    ("d128_c_1k", 128, True, [1024] * 4, 16, 4, "13"),
    ("d256_c_many", 256, True, [256] * 64, 8, 2, "13"),
    ("d256_c_round", 256, True, [256] * 16, 8, 2, "13"),
    ("d256_n_few", 256, False, [300, 290], 4, 2, "13"),
]


@pytest.mark.parametrize("case", DEFAULT_BRANCHES, ids=[c[0] for c in DEFAULT_BRANCHES])
def test_default_selection_branches(case):
    name, d, causal, lens, hq, hkv, expect = case
    assert "ATTN_FWD_TILE" not in os.environ
    t = api()
    w = gen.make_varlen(name, 1400 + d + len(lens), lens, hq, hkv, d, causal)
    ws = t.workspace(len(lens), w.max_seqlen, hq, d, causal)
    o, lse = t.attn_fwd_varlen(dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v),
                               dev_i32(w.cu_seqlens_q), dev_i32(w.cu_seqlens_k), w.max_seqlen,
                               scale=float(w.scale), causal=causal, workspace=ws)
    # the same call with the expected policy forced gives bit-identical output
    os.environ["ATTN_FWD_TILE"] = expect
    try:
        o2, lse2 = t.attn_fwd_varlen(dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v),
                                     dev_i32(w.cu_seqlens_q), dev_i32(w.cu_seqlens_k),
                                     w.max_seqlen, scale=float(w.scale), causal=causal,
                                     workspace=ws)
    finally:
        os.environ.pop("ATTN_FWD_TILE", None)
    o, lse, o2, lse2 = host(o), host(lse), host(o2), host(lse2)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2), "default differs from policy " + expect
    o_ref, lse_ref = oracle.attention_varlen(w.q, w.k, w.v, w.cu_seqlens_q, w.cu_seqlens_k,
                                             w.scale, causal)
    print(name, check_o(o, o_ref), check_lse(lse, lse_ref))


# Packs with one long sequence among many short ones (and empty ones): the
# (sequence, head) x longest-block-count grid would be mostly empty, so the
# library switches to the compact block order (one slot per real block).
# The host rule (rows x blocks >= 4 x heads x (ceil(total_q / bm) + nseq))
# holds for every case here with the default policy named in the comment.
SKEWED_PACKS = [
    ("d128_c", 128, True, [1500] + [20] * 60, 8, 2),         # 19, 256-query blocks
    ("d128_n", 128, False, [20] * 30 + [1500] + [20] * 30, 8, 2),  # 19
    ("d64_c_h12", 64, True, [1500] + [20] * 60 + [0, 0], 12, 4),   # 13, heads not a multiple of 8
    ("d64_n_h12", 64, False, [0] + [20] * 60 + [1500], 12, 4),     # 13
    ("d32_c", 32, True, [7] * 60 + [1500, 3], 8, 8),          # 19
]


@pytest.mark.parametrize("case", SKEWED_PACKS, ids=[c[0] for c in SKEWED_PACKS])
def test_compact_block_order_skewed_pack(case):
    name, d, causal, lens, hq, hkv = case
    assert "ATTN_FWD_TILE" not in os.environ
    w = gen.make_varlen("skew" + name, 1700 + d + hq, lens, hq, hkv, d, causal)
    t = api()
    plan = t.attn_fwd_launch_plan(True, len(lens), sum(lens), w.max_seqlen, hq, d, causal)
    assert plan["order"] == 4, plan  # the compact order is what runs by default
    o, lse = run_varlen(w)
    o_ref, lse_ref = oracle.attention_varlen(w.q, w.k, w.v, w.cu_seqlens_q, w.cu_seqlens_k,
                                             w.scale, causal)
    print(name, check_o(o, o_ref), check_lse(lse, lse_ref))
    # the same blocks in the order the pack would take without the compact
    # rule (sequence-major with hq % 8 == 0, else unit-major): bit-identical
    other = "2" if hq % 8 == 0 else "3"
    os.environ["ATTN_FWD_ORDER"] = other
    try:
        assert t.attn_fwd_launch_plan(True, len(lens), sum(lens), w.max_seqlen, hq, d,
                                      causal)["order"] == int(other)
        o2, lse2 = run_varlen(w)
    finally:
        os.environ.pop("ATTN_FWD_ORDER", None)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_compact_block_order_fused_padded():
    """The fused padded call on a skewed pack (compact order) equals the
    three-call path bit for bit and matches the oracle."""
    t = api()
    r = np.random.Generator(np.random.PCG64(1750))
    hq, hkv, d = 8, 2, 128
    slots = [2048] + [32] * 60
    lens = [1500] + [r.integers(0, 33) for _ in range(60)]
    total = sum(slots)
    mask = np.zeros(total, bool)
    st = 0
    for sl, L in zip(slots, lens):
        mask[st:st + L] = True
        st += sl
    idx_h = np.flatnonzero(mask).astype(np.int32)
    nz = [int(L) for L in lens if L > 0]
    cu_h = gen.cu_seqlens_from_lengths(nz)
    q = gen.normal_bf16(r, (1, total, hq, d))
    k = gen.normal_bf16(r, (1, total, hkv, d))
    v = gen.normal_bf16(r, (1, total, hkv, d))
    scale = 1.0 / math.sqrt(d)
    assert t.attn_fwd_launch_plan(True, len(nz), int(sum(nz)), max(nz), hq, d, True)["order"] == 4
    idx, cu = dev_i32(idx_h), dev_i32(cu_h)
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    pf, lsef = t.attn_fwd_padded(qd, kd, vd, idx, cu, max(nz), scale=scale, causal=True)
    (qc,) = t.attn_unpad_gather([qd], idx)  # q has more heads than k / v
    kc, vc = t.attn_unpad_gather([kd, vd], idx)
    o3, lse3 = t.attn_fwd_varlen(qc, kc, vc, cu, cu, max(nz), scale=scale, causal=True)
    p3 = host(t.attn_pad_scatter(o3, idx, total, out_shape=(1, total, hq, d)))
    pf = host(pf)
    assert np.array_equal(pf.view(np.uint32), p3.view(np.uint32))
    assert np.array_equal(host(lsef).view(np.uint32), host(lse3).view(np.uint32))
    qg = [oracle.unpad_gather(x, idx_h, x.shape[2:]) for x in (q, k, v)]
    o_ref, lse_ref = oracle.attention_varlen(qg[0], qg[1], qg[2], cu_h, cu_h, scale, True)
    check_o(host(o3), o_ref)
    check_lse(host(lse3), lse_ref)


# ----------------------------------------------------------------------------- gather / scatter
def test_gather_scatter_bit_exact_with_nan_bits_and_bad_index():
    import torch
    t = api()
    r = np.random.Generator(np.random.PCG64(1100))
    n_rows, hd = 300, (3, 40)
    srcs = [r.integers(0, 2 ** 16, size=(n_rows,) + hd, dtype=np.uint16) for _ in range(3)]
    srcs[0][5] = 0x7FC1  # NaN bit patterns copy unchanged
    idx = np.sort(r.choice(n_rows, size=123, replace=False)).astype(np.int32)
    outs = t.attn_unpad_gather([dev_bf16(s) for s in srcs], dev_i32(idx))
    for s, o in zip(srcs, outs):
        assert np.array_equal(host(o), oracle.unpad_gather(s, idx, hd))
    back = t.attn_pad_scatter(outs[1], dev_i32(idx), n_rows)
    assert np.array_equal(host(back), oracle.pad_scatter(oracle.unpad_gather(srcs[1], idx, hd),
                                                         idx, n_rows))
    # an out-of-range gather index yields a zero row, never a fault
    bad = idx.copy()
    bad[7] = n_rows + 5
    bad[8] = -3
    o1 = t.attn_unpad_gather([dev_bf16(srcs[2])], dev_i32(bad))[0]
    h1 = host(o1)
    assert np.all(h1[7] == 0) and np.all(h1[8] == 0)
    keep = np.ones(len(idx), bool)
    keep[[7, 8]] = False
    assert np.array_equal(h1[keep], srcs[2][idx[keep]])
    # fp32 rows too (the scatter's main use is the fp32 attention output)
    f = torch.randn(123, 16, 32, device="cuda")
    fs = t.attn_pad_scatter(f, dev_i32(idx), n_rows)
    assert np.array_equal(host(fs), oracle.pad_scatter(host(f), idx, n_rows))


@pytest.mark.parametrize("n_valid,n_rows", [(0, 50), (1, 1), (4096, 4096), (2000, 65536), (7, 9)])
def test_scatter_search_sizes(n_valid, n_rows):
    import torch
    t = api()
    r = np.random.Generator(np.random.PCG64(1200 + n_rows))
    idx = np.sort(r.choice(n_rows, size=n_valid, replace=False)).astype(np.int32)
    src = torch.randn(n_valid, 4, 4, device="cuda")
    out = t.attn_pad_scatter(src, dev_i32(idx), n_rows)
    assert np.array_equal(host(out), oracle.pad_scatter(host(src), idx, n_rows))


# ----------------------------------------------------------------------------- split key ranges
SPLIT_POLICIES = ["11", "12", "13", "17", "19"]


def _forced_split(policy, tiles):
    os.environ["ATTN_FWD_TILE"] = policy
    os.environ["ATTN_FWD_SPLIT_TILES"] = str(tiles)


def _clear_forced():
    os.environ.pop("ATTN_FWD_TILE", None)
    os.environ.pop("ATTN_FWD_SPLIT_TILES", None)


@pytest.mark.parametrize("policy", SPLIT_POLICIES)
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("d", [32, 64, 128, 256])
def test_split_key_ranges_varlen(policy, causal, d):
    """Key loops cut into parts of 1-3 tiles (several parts per block, uneven
    last parts, empty sequences, GQA) and merged, against the oracle."""
    if not compiled(policy, d):
        pytest.skip("policy not compiled for this head_dim")
    t = api()
    w = gen.make_varlen("split", 1500 + d, [150, 64, 1, 0, 90, 700, 333], 4, 2, d, causal)
    for tiles in (1, 3):
        _forced_split(policy, tiles)
        try:
            ws = t.workspace(len(w.lengths_q), w.max_seqlen, 4, d, causal)
            assert ws is not None
            o, lse = t.attn_fwd_varlen(dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v),
                                       dev_i32(w.cu_seqlens_q), dev_i32(w.cu_seqlens_k),
                                       w.max_seqlen, scale=float(w.scale), causal=causal,
                                       workspace=ws)
        finally:
            _clear_forced()
        o_ref, lse_ref = oracle.attention_varlen(w.q, w.k, w.v, w.cu_seqlens_q, w.cu_seqlens_k,
                                                 w.scale, causal)
        print(policy, d, causal, tiles, check_o(host(o), o_ref), check_lse(host(lse), lse_ref))


@pytest.mark.parametrize("policy", SPLIT_POLICIES)
def test_split_key_ranges_dense_lq_ne_lk(policy):
    """Dense, bottom-right causal with Lk > Lq and Lk < Lq, strided output."""
    t = api()
    for sq, sk in ((300, 520), (520, 300)):
        w = gen.make_dense(f"sd{sq}", 1600 + sq, 2, sq, sk, 4, 1, 128, True)
        _forced_split(policy, 2)
        try:
            ws = t.workspace(2, sq, 4, 128, True)
            o, lse = t.attn_fwd_dense(dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v),
                                      scale=float(w.scale), causal=True, workspace=ws)
        finally:
            _clear_forced()
        o_ref, lse_ref = oracle.attention_dense(w.q, w.k, w.v, w.scale, True)
        print(policy, sq, sk, check_o(host(o), o_ref), check_lse(host(lse), lse_ref))


def test_split_workspace_too_small_runs_unsplit():
    import torch
    t = api()
    w = gen.make_varlen("small", 1700, [700, 300], 2, 2, 128, True)
    _forced_split("12", 2)
    try:
        n = t.attn_fwd_workspace_bytes(2, w.max_seqlen, 2, 128, True)
        assert n > 0
        small = torch.empty(n - 16, dtype=torch.uint8, device="cuda")
        o, lse = t.attn_fwd_varlen(dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v),
                                   dev_i32(w.cu_seqlens_q), dev_i32(w.cu_seqlens_k),
                                   w.max_seqlen, scale=float(w.scale), causal=True,
                                   workspace=small)
    finally:
        _clear_forced()
    o_ref, lse_ref = oracle.attention_varlen(w.q, w.k, w.v, w.cu_seqlens_q, w.cu_seqlens_k,
                                             w.scale, True)
    check_o(host(o), o_ref)
    check_lse(host(lse), lse_ref)


# ----------------------------------------------------------------------------- the padded path end to end
@pytest.mark.parametrize("name,use_ws", [("padded_32x128_random", False),
                                         ("padded_32x128_exact", False),
                                         ("padded_1x2048", False), ("padded_1x2048", True)])
def test_padded_path_full_size(name, use_ws):
    t = api()
    w = gen.build_workload(name)
    idx = dev_i32(w.indices)
    qc, kc, vc = t.attn_unpad_gather([dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)], idx)
    ws = None
    if use_ws:  # split path at full size: policy 12, parts of at most 8 key tiles
        os.environ["ATTN_FWD_TILE"] = "12"
        os.environ["ATTN_FWD_SPLIT_TILES"] = "8"
    try:
        if use_ws:
            ws = t.workspace(len(w.lengths_q), w.max_seqlen, w.hq, w.d, True)
            assert ws is not None
        o, lse = t.attn_fwd_varlen(qc, kc, vc, dev_i32(w.cu_seqlens_q), dev_i32(w.cu_seqlens_k),
                                   w.max_seqlen, scale=float(w.scale), causal=True, workspace=ws)
    finally:
        os.environ.pop("ATTN_FWD_SPLIT_TILES", None)
        os.environ.pop("ATTN_FWD_TILE", None)
    padded = t.attn_pad_scatter(o, idx, w.q.shape[1], out_shape=(1,) + w.q.shape[1:])
    # the oracle: gather, attention, scatter
    hd = w.q.shape[2:]
    gq, gk, gv = (oracle.unpad_gather(x, w.indices, hd) for x in (w.q, w.k, w.v))
    assert np.array_equal(host(qc), gq) and np.array_equal(host(kc), gk)
    o_ref, lse_ref = oracle.attention_varlen(gq, gk, gv, w.cu_seqlens_q, w.cu_seqlens_k, w.scale, True)
    p_ref = oracle.pad_scatter(o_ref, w.indices, w.q.shape[1]).reshape((1,) + w.q.shape[1:])
    ph = host(padded)
    pad_rows = np.ones(w.q.shape[1], bool)
    pad_rows[w.indices] = False
    assert np.all(ph[0, pad_rows].view(np.uint32) == 0)  # +0.0 bits
    print(check_o(ph, p_ref), check_lse(host(lse), lse_ref))


# ----------------------------------------------------------------------------- fused padded path
@pytest.mark.parametrize("name", ["padded_32x128_random", "padded_32x128_exact", "padded_1x2048"])
def test_fused_padded_equals_three_call_path_bitwise(name):
    """attn_fwd_padded reads and writes the padded rows in place; with the
    same tile policy it computes exactly what gather + varlen + scatter do."""
    t = api()
    w = gen.build_workload(name)
    idx = dev_i32(w.indices)
    cu = dev_i32(w.cu_seqlens_q)
    q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    qc, kc, vc = t.attn_unpad_gather([q, k, v], idx)
    o3, lse3 = t.attn_fwd_varlen(qc, kc, vc, cu, cu, w.max_seqlen, scale=float(w.scale),
                                 causal=True)
    p3 = host(t.attn_pad_scatter(o3, idx, w.q.shape[1], out_shape=(1,) + w.q.shape[1:]))
    pf, lsef = t.attn_fwd_padded(q, k, v, idx, cu, w.max_seqlen, scale=float(w.scale),
                                 causal=True)
    pf = host(pf)
    assert pf.shape == p3.shape
    assert np.array_equal(pf.view(np.uint32), p3.view(np.uint32))
    assert np.array_equal(host(lsef).view(np.uint32), host(lse3).view(np.uint32))
    pad_rows = np.ones(w.q.shape[1], bool)
    pad_rows[w.indices] = False
    assert np.all(pf[0, pad_rows].view(np.uint32) == 0)


@pytest.mark.parametrize("d", [64, 128])
def test_fused_padded_gqa_nan_padding_vs_oracle(d):
    """Grouped heads, NaN in every padding row of q/k/v, slots of mixed
    lengths with an empty one; compared with the oracle's gather, attention
    and scatter."""
    t = api()
    r = np.random.Generator(np.random.PCG64(1800 + d))
    total, hq, hkv = 1536, 4, 2
    slots = [256, 512, 128, 384, 256]
    lens = [200, 512, 0, 1, 97]
    mask = np.zeros(total, bool)
    st = 0
    for sl, L in zip(slots, lens):
        mask[st:st + L] = True
        st += sl
    idx = np.flatnonzero(mask).astype(np.int32)
    nz = [L for L in lens if L > 0]
    cu = gen.cu_seqlens_from_lengths(nz)
    nan = gen.bf16_bits_from_f32(np.array([np.nan], np.float32))[0]
    q = gen.normal_bf16(r, (1, total, hq, d))
    k = gen.normal_bf16(r, (1, total, hkv, d))
    v = gen.normal_bf16(r, (1, total, hkv, d))
    for x in (q, k, v):
        x[0, ~mask] = nan
    for causal in (True, False):
        out, lse = t.attn_fwd_padded(dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_i32(idx),
                                     dev_i32(cu), max(nz), causal=causal)
        out = host(out)
        assert not np.isnan(out).any()
        assert np.all(out[0, ~mask].view(np.uint32) == 0)
        gq = oracle.unpad_gather(q, idx, (hq, d))
        gk = oracle.unpad_gather(k, idx, (hkv, d))
        gv = oracle.unpad_gather(v, idx, (hkv, d))
        scale = np.float32(1.0 / math.sqrt(d))
        o_ref, lse_ref = oracle.attention_varlen(gq, gk, gv, cu, cu, scale, causal)
        p_ref = oracle.pad_scatter(o_ref, idx, total).reshape(out.shape)
        print(d, causal, check_o(out, p_ref), check_lse(host(lse), lse_ref))


def test_fused_padded_all_padding_is_zero_fill():
    import torch
    t = api()
    q = torch.full((1, 256, 2, 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty(0, dtype=torch.int32, device="cuda")
    cu = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.full((1, 256, 2, 64), 5.0, dtype=torch.float32, device="cuda")
    t.attn_fwd_padded(q, q, q, idx, cu, 0, causal=True, out=out, return_lse=False)
    assert np.all(host(out).view(np.uint32) == 0)


def test_padded_path_nan_padding_does_not_leak():
    t = api()
    w = gen.make_padded("nan", 1300, 1024, [128] * 8, 4, 64, True, random_max=128,
                        pad_value=float("nan"))
    idx = dev_i32(w.indices)
    qc, kc, vc = t.attn_unpad_gather([dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)], idx)
    o, lse = t.attn_fwd_varlen(qc, kc, vc, dev_i32(w.cu_seqlens_q), dev_i32(w.cu_seqlens_k),
                               w.max_seqlen, scale=float(w.scale), causal=True)
    padded = host(t.attn_pad_scatter(o, idx, 1024))
    assert not np.isnan(padded).any()
    hd = w.q.shape[2:]
    gq, gk, gv = (oracle.unpad_gather(x, w.indices, hd) for x in (w.q, w.k, w.v))
    o_ref, _ = oracle.attention_varlen(gq, gk, gv, w.cu_seqlens_q, w.cu_seqlens_k, w.scale, True)
    check_o(padded, oracle.pad_scatter(o_ref, w.indices, 1024))


# ----------------------------------------------------------------------------- HIP graph capture
def test_padded_path_graph_replays_match_eager():
    """The three launches are capturable: every replay (with eager work and
    synchronisations in between) reproduces the eager result bit for bit."""
    import torch
    t = api()
    w = gen.make_padded("graph", 1400, 1024, [256] * 4, 4, 128, True, random_max=256)
    idx = dev_i32(w.indices)
    cu = dev_i32(w.cu_seqlens_q)
    q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    n = len(w.indices)
    qc, kc, vc = (torch.empty((n, 4, 128), dtype=torch.bfloat16, device="cuda") for _ in range(3))
    o = torch.empty((n, 4, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((4, n), dtype=torch.float32, device="cuda")
    out = torch.empty((1, 1024, 4, 128), dtype=torch.float32, device="cuda")

    def step():
        t.attn_unpad_gather([q, k, v], idx, outs=[qc, kc, vc])
        t.attn_fwd_varlen(qc, kc, vc, cu, cu, w.max_seqlen, scale=float(w.scale), causal=True,
                          out=o, lse=lse)
        t.attn_pad_scatter(o, idx, 1024, out=out)

    step()
    torch.cuda.synchronize()
    ref_out, ref_lse = host(out).copy(), host(lse).copy()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for i in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out), ref_out), f"replay {i}"
        assert np.array_equal(host(lse), ref_lse), f"replay {i}"
        step()  # eager work between replays
        torch.cuda.synchronize()
