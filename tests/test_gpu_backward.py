"""GPU parity of the attention backward: the HIP path through the C ABI
against the fp64 gradient oracle.

Each case runs the library's forward (out, lse) and then its backward on the
same seeded bf16 inputs, and compares dq, dk, dv with the oracle's exact
gradients of the attention definition.  Sizes span several 128-row blocks and
64-row tiles with ragged tails; GQA, Lq != Lk, empty sequences and queries that
see no key are covered.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from synth import gen
from tests.gpu_util import check_grad, dev_bf16, dev_i32, host

pytestmark = pytest.mark.gpu


def api():
    import tiled_attention_fwd_amd as t
    return t


def run_varlen_bwd(w, do_bits, causal=None):
    t = api()
    causal = w.causal if causal is None else causal
    q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    cq, ck = dev_i32(w.cu_seqlens_q), dev_i32(w.cu_seqlens_k)
    mq = max(w.lengths_q + [0])
    mk = max(w.lengths_k + [0])
    out, lse = t.attn_fwd_varlen(q, k, v, cq, ck, max(mq, 1), scale=float(w.scale), causal=causal)
    dq, dk, dv = t.attn_bwd_varlen(q, k, v, out, lse, dev_bf16(do_bits), cq, ck, max(mq, 1),
                                   max(mk, 1), scale=float(w.scale), causal=causal)
    return host(dq), host(dk), host(dv)


def run_dense_bwd(w, do_bits):
    t = api()
    q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    out, lse = t.attn_fwd_dense(q, k, v, scale=float(w.scale), causal=w.causal)
    dq, dk, dv = t.attn_bwd_dense(q, k, v, out, lse, dev_bf16(do_bits), scale=float(w.scale),
                                  causal=w.causal)
    return host(dq), host(dk), host(dv)


def compare(got, ref, tag):
    res = {}
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        res[name] = check_grad(g, r, f"{tag}:{name}")
    print(tag, res)
    return res


@pytest.mark.parametrize("d", [32, 64, 128, 256])
@pytest.mark.parametrize("causal", [True, False])
def test_bwd_varlen_ragged_gqa(d, causal):
    lens = [1, 7, 64, 100, 129, 300, 33]
    w = gen.make_varlen(f"bvr{d}", 600 + d, lens, 4, 2, d, causal)
    do = gen.upstream_grad_bf16(w.seed, w.q.shape)
    got = run_varlen_bwd(w, do)
    ref = oracle.attention_backward_varlen(w.q, w.k, w.v, do, w.cu_seqlens_q, w.cu_seqlens_k,
                                           w.scale, causal)
    compare(got, ref, f"varlen d={d} causal={causal}")


@pytest.mark.parametrize("d", [32, 64, 128, 256])
@pytest.mark.parametrize("causal", [True, False])
def test_bwd_varlen_lq_ne_lk_and_empty(d, causal):
    lq = [5, 130, 0, 64, 3, 0, 200]
    lk = [9, 70, 12, 200, 0, 0, 257]
    w = gen.make_varlen("bne", 700 + d, lq, 2, 2, d, causal, lengths_k=lk)
    do = gen.upstream_grad_bf16(w.seed, w.q.shape)
    got = run_varlen_bwd(w, do)
    ref = oracle.attention_backward_varlen(w.q, w.k, w.v, do, w.cu_seqlens_q, w.cu_seqlens_k,
                                           w.scale, causal)
    compare(got, ref, f"lq!=lk d={d} causal={causal}")
    # keys of a sequence without queries get zero gradients, exactly
    ck = w.cu_seqlens_k
    assert np.all(got[1][ck[2]:ck[3]] == 0.0) and np.all(got[2][ck[2]:ck[3]] == 0.0)


@pytest.mark.parametrize("d", [32, 64, 128, 256])
@pytest.mark.parametrize("causal", [True, False])
def test_bwd_dense(d, causal):
    w = gen.make_dense(f"bdn{d}", 800 + d, 2, 200, 200, 4, 1, d, causal)
    do = gen.upstream_grad_bf16(w.seed, w.q.shape)
    got = run_dense_bwd(w, do)
    ref = oracle.attention_backward_dense(w.q, w.k, w.v, do, w.scale, causal)
    compare(got, ref, f"dense d={d} causal={causal}")


@pytest.mark.parametrize("causal", [True, False])
def test_bwd_dense_sq_ne_sk(causal):
    w = gen.make_dense("bdne", 901, 1, 96, 333, 2, 2, 128, causal)
    do = gen.upstream_grad_bf16(w.seed, w.q.shape)
    got = run_dense_bwd(w, do)
    ref = oracle.attention_backward_dense(w.q, w.k, w.v, do, w.scale, causal)
    compare(got, ref, f"dense 96x333 causal={causal}")


def test_bwd_varlen_1x2048_sampled_heads():
    """The 1 x 2048, 16-head, d=128 causal shape at full size; the oracle
    computes two of the heads (heads are independent when Hq == Hkv)."""
    w = gen.make_varlen("b2048", 950, [2048], 16, 16, 128, True)
    do = gen.upstream_grad_bf16(w.seed, w.q.shape)
    got = run_varlen_bwd(w, do)
    for h in (0, 11):
        sl = slice(h, h + 1)
        ref = oracle.attention_backward_varlen(w.q[:, sl], w.k[:, sl], w.v[:, sl], do[:, sl],
                                               w.cu_seqlens_q, w.cu_seqlens_k, w.scale, True)
        compare([g[:, sl] for g in got], ref, f"1x2048 head {h}")


def test_bwd_deterministic():
    w = gen.make_varlen("bdet", 960, [300, 77], 4, 1, 128, True)
    do = gen.upstream_grad_bf16(w.seed, w.q.shape)
    a = run_varlen_bwd(w, do)
    b = run_varlen_bwd(w, do)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_bwd_rejects_unsupported_head_dim():
    import torch
    t = api()
    q = torch.zeros((40, 2, 48), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((40, 2, 48), dtype=torch.float32, device="cuda")
    lse = torch.zeros((2, 40), dtype=torch.float32, device="cuda")
    cq = dev_i32(np.array([0, 40], dtype=np.int32))
    with pytest.raises(t.AttnError, match="UNSUPPORTED"):
        t.attn_bwd_varlen(q, q, q, out, lse, q, cq, cq, 40)
