"""GPU parity at zero and negative score scales (every finite scale is valid).

The definition softmax(scale * Q K^T) V (page "Intro to FlashAttention on
Ascend CANN", section on the traditional implementation, which uses the scale
1/sqrt(d_k)) holds for any finite scale: a zero scale gives every visible key
the same weight (the output is the mean of the visible value rows and the LSE
is ln of their count), a negative one weights the smallest dot products
highest.  Each case compares the library with the fp64 oracle; two exact
identities are checked bit for bit on the GPU:
  * scale 0 on (Q, K, V) equals scale s > 0 on (0, K, V) (all scores exactly 0);
  * scale -s on (Q, K, V) equals scale s on (-Q, K, V) (bf16 negation is exact).
"""

from __future__ import annotations

import math
import os

import numpy as np
import pytest

import oracle
from synth import gen
from tests.gpu_util import check_grad, check_lse, check_o, dev_bf16, dev_i32, host
from tests.test_gpu_fp8 import check_fp8

pytestmark = pytest.mark.gpu

D_ALL = [32, 64, 128, 256]


def api():
    import tiled_attention_fwd_amd as t
    return t


def varlen(w, scale, q=None, **kw):
    t = api()
    o, lse = t.attn_fwd_varlen(dev_bf16(w.q if q is None else q), dev_bf16(w.k), dev_bf16(w.v),
                               dev_i32(w.cu_seqlens_q), dev_i32(w.cu_seqlens_k), w.max_seqlen,
                               scale=scale, causal=w.causal, **kw)
    return host(o), host(lse)


def oracle_varlen(w, scale):
    return oracle.attention_varlen(w.q, w.k, w.v, w.cu_seqlens_q, w.cu_seqlens_k,
                                   np.float32(scale), w.causal)


def neg_bits(bits):
    return bits ^ np.uint16(0x8000)


@pytest.mark.parametrize("policy", [str(i) for i in range(21)])
def test_every_policy_negative_and_zero_scale(policy):
    """Every compiled tile policy, every head_dim, causal and not."""
    t = api()
    os.environ["ATTN_FWD_TILE"] = policy
    try:
        ran = 0
        for d in D_ALL:
            if not t.attn_fwd_tile_policy_compiled(int(policy), d):
                continue
            for causal, scale in ((True, -1.0 / math.sqrt(d)), (False, 0.0), (True, 0.0),
                                  (False, -0.3)):
                w = gen.make_varlen("neg", 2100 + d, [150, 64, 1, 90, 300], 2, 1, d, causal)
                o, lse = varlen(w, scale)
                o_ref, lse_ref = oracle_varlen(w, scale)
                check_o(o, o_ref, f"policy {policy} d={d} causal={causal} scale={scale}")
                check_lse(lse, lse_ref, f"policy {policy} d={d} causal={causal} scale={scale}")
                ran += 1
        if ran == 0:
            pytest.skip("policy not compiled for any head_dim")
    finally:
        del os.environ["ATTN_FWD_TILE"]


@pytest.mark.parametrize("d", D_ALL)
@pytest.mark.parametrize("causal", [True, False])
def test_zero_scale_closed_form_and_zero_query_identity(d, causal):
    """Scale 0: out is the mean of the visible value rows, lse = ln(count), and
    the result equals the positive-scale call on Q = 0 bit for bit."""
    lens = [700, 33, 1, 260]
    w = gen.make_varlen("zs", 2200 + d, lens, 4, 2, d, causal)
    o, lse = varlen(w, 0.0)
    oz, lz = varlen(w, 1.0 / math.sqrt(d), q=np.zeros_like(w.q))
    assert np.array_equal(o.view(np.uint32), oz.view(np.uint32))
    assert np.array_equal(lse.view(np.uint32), lz.view(np.uint32))
    v = oracle.bf16_bits_to_f64(w.v)
    cq = w.cu_seqlens_q
    o_cf = np.zeros(o.shape)
    l_cf = np.zeros(lse.shape)
    for s, L in enumerate(lens):
        vs = v[cq[s]:cq[s + 1]]
        cnt = np.arange(1, L + 1) if causal else np.full(L, L)
        means = (np.cumsum(vs, axis=0) / cnt[:, None, None]) if causal else \
            np.broadcast_to(vs.mean(axis=0), vs.shape)
        for h in range(w.hq):
            o_cf[cq[s]:cq[s + 1], h] = means[:, h // 2]
            l_cf[h, cq[s]:cq[s + 1]] = np.log(cnt)
    check_o(o, o_cf, "closed form")
    check_lse(lse, l_cf, "closed form")


@pytest.mark.parametrize("d", D_ALL)
def test_negative_scale_equals_negated_query(d):
    w = gen.make_varlen("ns", 2300 + d, [1200, 5, 333], 8, 2, d, True)
    s = 1.0 / math.sqrt(d)
    o, lse = varlen(w, -s)
    o2, l2 = varlen(w, s, q=neg_bits(w.q))
    assert np.array_equal(o.view(np.uint32), o2.view(np.uint32))
    assert np.array_equal(lse.view(np.uint32), l2.view(np.uint32))
    o_ref, lse_ref = oracle_varlen(w, -s)
    check_o(o, o_ref)
    check_lse(lse, lse_ref)


@pytest.mark.parametrize("scale", [-0.0883883, 0.0])
def test_dense_split_and_padded_paths(scale):
    t = api()
    # dense, grouped heads, bottom-right causal with Lq != Lk
    w = gen.make_dense("nd", 2400, 2, 200, 333, 8, 2, 128, True)
    o, lse = t.attn_fwd_dense(dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v), scale=scale,
                              causal=True)
    o_ref, lse_ref = oracle.attention_dense(w.q, w.k, w.v, np.float32(scale), True)
    check_o(host(o), o_ref)
    check_lse(host(lse), lse_ref)
    # split key ranges (forced 2-tile parts of policy 19's 128-key tiles)
    wv = gen.make_varlen("nsplit", 2401, [2048], 2, 2, 128, True)
    os.environ["ATTN_FWD_SPLIT_TILES"] = "2"
    os.environ["ATTN_FWD_TILE"] = "19"
    try:
        ws = t.workspace(1, 2048, 2, 128, True)
        assert ws is not None
        o, lse = varlen(wv, scale, workspace=ws)
    finally:
        os.environ.pop("ATTN_FWD_SPLIT_TILES", None)
        os.environ.pop("ATTN_FWD_TILE", None)
    o_ref, lse_ref = oracle_varlen(wv, scale)
    check_o(o, o_ref)
    check_lse(lse, lse_ref)
    # fused padded call
    wp = gen.make_padded("npad", 2402, 1024, [256] * 4, 4, 64, True, random_max=256,
                         pad_value=float("nan"))
    out, lse = t.attn_fwd_padded(dev_bf16(wp.q), dev_bf16(wp.k), dev_bf16(wp.v),
                                 dev_i32(wp.indices), dev_i32(wp.cu_seqlens_q), wp.max_seqlen,
                                 scale=scale, causal=True)
    out = host(out)
    g = [oracle.unpad_gather(x, wp.indices, x.shape[2:]) for x in (wp.q, wp.k, wp.v)]
    o_ref, lse_ref = oracle.attention_varlen(*g, wp.cu_seqlens_q, wp.cu_seqlens_k,
                                             np.float32(scale), True)
    check_o(out, oracle.pad_scatter(o_ref, wp.indices, 1024).reshape(out.shape))
    check_lse(host(lse), lse_ref)


@pytest.mark.parametrize("scale", [-0.0883883, 0.0])
def test_fp8_paged_and_backward(scale):
    import torch
    t = api()
    # fp8 inputs
    w8 = gen.make_fp8_varlen("n8", 2500, [300, 7, 129], 4, 2, 128, True, factors=(2.0, 0.5, 1.0))
    u8 = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).to("cuda")
    o, lse = t.attn_fwd_fp8_varlen(u8(w8.q), u8(w8.k), u8(w8.v), dev_i32(w8.cu_seqlens_q),
                                   dev_i32(w8.cu_seqlens_k), w8.max_seqlen, scale=scale,
                                   q_scale=float(w8.q_scale), k_scale=float(w8.k_scale),
                                   v_scale=float(w8.v_scale), causal=True)
    # the fp8 tests' per-element bound (E4M3 probabilities), at this scale
    w8.scale = np.float32(scale)
    check_fp8(w8, host(o), host(lse), True)
    # paged KV cache
    wp = gen.make_paged("npg", 2501, [1, 4, 3], [300, 33, 200], 8, 2, 128, 32, True,
                        fill=float("nan"))
    o, lse = t.attn_fwd_paged(dev_bf16(wp.q), dev_bf16(wp.k_cache), dev_bf16(wp.v_cache),
                              dev_i32(wp.cu_seqlens_q), dev_i32(wp.seqlens_k),
                              dev_i32(wp.block_table), wp.max_seqlen_q, wp.max_seqlen_k,
                              scale=scale, causal=True)
    o_ref, lse_ref = oracle.attention_paged(wp.q, wp.k_cache, wp.v_cache, wp.cu_seqlens_q,
                                            wp.seqlens_k, wp.block_table, np.float32(scale), True)
    check_o(host(o), o_ref, "paged")
    check_lse(host(lse), lse_ref, "paged")
    # backward through the library's own forward
    wb = gen.make_varlen("nb", 2502, [129, 64, 300], 4, 2, 64, True)
    do = gen.upstream_grad_bf16(wb.seed, wb.q.shape)
    q, k, v = dev_bf16(wb.q), dev_bf16(wb.k), dev_bf16(wb.v)
    cq, ck = dev_i32(wb.cu_seqlens_q), dev_i32(wb.cu_seqlens_k)
    out, lse = t.attn_fwd_varlen(q, k, v, cq, ck, wb.max_seqlen, scale=scale, causal=True)
    dq, dk, dv = t.attn_bwd_varlen(q, k, v, out, lse, dev_bf16(do), cq, ck, wb.max_seqlen,
                                   wb.max_seqlen, scale=scale, causal=True)
    ref = oracle.attention_backward_varlen(wb.q, wb.k, wb.v, do, wb.cu_seqlens_q, wb.cu_seqlens_k,
                                           np.float32(scale), True)
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        check_grad(host(g), r, f"backward {name}")
