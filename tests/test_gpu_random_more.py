"""Randomised GPU parity sweeps (seeded) for the paged KV cache, the fp8 path
and the backward, each against its fp64 oracle.  Shapes stay small enough for
the oracle and cover ragged lengths, empty sequences, grouped heads and both
causal settings; the paged cases also draw the page size and whether a split
workspace is passed, and fill every unowned cache row with NaN."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from synth import gen
from tests.gpu_util import check_grad, check_lse, check_o, dev_bf16, dev_i32, host

pytestmark = pytest.mark.gpu


def api():
    import tiled_attention_fwd_amd as t
    return t


@pytest.mark.parametrize("seed", range(8000, 8012))
def test_random_paged(seed):
    t = api()
    r = np.random.Generator(np.random.PCG64(seed))
    d = int(r.choice([64, 128]))
    hkv = int(r.choice([1, 2]))
    group = int(r.choice([1, 2, 4, 8]))
    nseq = int(r.integers(1, 6))
    page = int(r.choice([16, 32, 48, 64, 128]))
    lq = [int(r.choice([0, 1, 1, 2, 4, int(r.integers(1, 80))])) for _ in range(nseq)]
    if sum(lq) == 0:
        lq[0] = 1
    lk = [int(r.integers(0, 600)) for _ in range(nseq)]
    causal = bool(r.random() < 0.7)
    w = gen.make_paged(f"rp{seed}", seed, lq, lk, hkv * group, hkv, d, page, causal,
                       fill=float("nan"))
    ws = None
    if r.random() < 0.5 and w.max_seqlen_k > 0:
        ws = t.paged_workspace(nseq, max(w.max_seqlen_q, 1), w.max_seqlen_k, w.hq, hkv, d)
    o, lse = t.attn_fwd_paged(dev_bf16(w.q), dev_bf16(w.k_cache), dev_bf16(w.v_cache),
                              dev_i32(w.cu_seqlens_q), dev_i32(w.seqlens_k),
                              dev_i32(w.block_table), max(w.max_seqlen_q, 1), w.max_seqlen_k,
                              scale=float(w.scale), causal=causal, workspace=ws)
    o_ref, lse_ref = oracle.attention_paged(w.q, w.k_cache, w.v_cache, w.cu_seqlens_q,
                                            w.seqlens_k, w.block_table, w.scale, causal)
    check_o(host(o), o_ref)
    check_lse(host(lse), lse_ref)


@pytest.mark.parametrize("seed", range(8100, 8110))
def test_random_fp8(seed):
    t = api()
    r = np.random.Generator(np.random.PCG64(seed))
    d = int(r.choice([64, 128]))
    hkv = int(r.choice([1, 2]))
    hq = hkv * int(r.choice([1, 2, 4]))
    nseq = int(r.integers(1, 5))
    lq = [int(r.integers(0, 300)) for _ in range(nseq)]
    if sum(lq) == 0:
        lq[0] = 1
    lk = [a if r.random() < 0.6 else int(r.integers(0, 350)) for a in lq]
    causal = bool(r.random() < 0.6)
    f = tuple(float(2.0 ** int(r.integers(-2, 3))) for _ in range(3))
    w = gen.make_fp8_varlen(f"rf{seed}", seed, lq, hq, hkv, d, causal, lengths_k=lk, factors=f)
    u8 = lambda x: __import__("torch").from_numpy(np.ascontiguousarray(x)).to("cuda")
    o, lse = t.attn_fwd_fp8_varlen(u8(w.q), u8(w.k), u8(w.v), dev_i32(w.cu_seqlens_q),
                                   dev_i32(w.cu_seqlens_k), max(max(lq), 1), scale=float(w.scale),
                                   q_scale=f[0], k_scale=f[1], v_scale=f[2], causal=causal)
    o, lse = host(o), host(lse)
    args = (w.cu_seqlens_q, w.cu_seqlens_k, w.scale, *f, causal)
    o_ref, lse_ref = oracle.attention_fp8_varlen(w.q, w.k, w.v, *args)
    o_abs, _ = oracle.attention_fp8_varlen(w.q, w.k, w.v & np.uint8(0x7F), *args)
    vmax = float(np.abs(oracle.e4m3_to_f64(w.v)).max()) * f[2] if w.v.size else 0.0
    lk_row = np.zeros(o.shape[0])
    for s in range(nseq):
        lk_row[w.cu_seqlens_q[s]:w.cu_seqlens_q[s + 1]] = lk[s]
    bound = 2.0 ** -4 * o_abs + (2.0 ** -17 * lk_row * vmax)[:, None, None] + 1e-6
    assert np.isfinite(o).all()
    assert (np.abs(o - o_ref) <= bound).all()
    check_lse(lse, lse_ref)


@pytest.mark.parametrize("seed", range(8200, 8208))
def test_random_backward(seed):
    t = api()
    r = np.random.Generator(np.random.PCG64(seed))
    d = int(r.choice([64, 128]))
    hkv = int(r.choice([1, 2]))
    hq = hkv * int(r.choice([1, 2, 4]))
    nseq = int(r.integers(1, 5))
    lq = [int(r.integers(0, 300)) for _ in range(nseq)]
    if sum(lq) == 0:
        lq[0] = 1
    lk = [a if r.random() < 0.6 else int(r.integers(0, 350)) for a in lq]
    causal = bool(r.random() < 0.6)
    w = gen.make_varlen(f"rb{seed}", seed, lq, hq, hkv, d, causal, lengths_k=lk)
    do = gen.upstream_grad_bf16(seed, w.q.shape)
    q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    cq, ck = dev_i32(w.cu_seqlens_q), dev_i32(w.cu_seqlens_k)
    mq, mk = max(max(lq), 1), max(max(lk), 1)
    out, lse = t.attn_fwd_varlen(q, k, v, cq, ck, mq, scale=float(w.scale), causal=causal)
    dq, dk, dv = t.attn_bwd_varlen(q, k, v, out, lse, dev_bf16(do), cq, ck, mq, mk,
                                   scale=float(w.scale), causal=causal)
    ref = oracle.attention_backward_varlen(w.q, w.k, w.v, do, w.cu_seqlens_q, w.cu_seqlens_k,
                                           w.scale, causal)
    for name, g, rr in zip(("dq", "dk", "dv"), (host(dq), host(dk), host(dv)), ref):
        check_grad(g, rr, f"seed {seed} {name}")
