"""GPU parity of the fp8 (E4M3) attention against oracle.attention_fp8_*.

Bar (derived from the one rounding the kernel adds): the scores and row sums
are exact fp8 products accumulated in fp32, and the probabilities enter the
P*V product as E4M3 bytes of 2^7 p (p relative to the row's running reference,
at most 2, and the row sum l >= 1 in the same units).  In the normal range
that rounding is at most 2^-4 of p; below it (2^7 p < 2^-6) at most 2^-17
absolute.  So, per output element, |O - O_ref| <= 2^-4 * sum_k p_k |v_k| / l +
2^-17 * Lk * max|v| (+ 1e-6 for fp32 accumulation), where sum_k p_k |v_k| / l
is the oracle's own output for |v| (sign bits cleared).  LSE: |dLSE| <= 1e-3 as
for bf16.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from synth import gen
from tests.gpu_util import check_lse, dev_i32, host

pytestmark = pytest.mark.gpu


def api():
    import tiled_attention_fwd_amd as t
    return t


def dev_u8(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).to("cuda")


def run_varlen(w, causal=None):
    t = api()
    causal = w.causal if causal is None else causal
    o, lse = t.attn_fwd_fp8_varlen(dev_u8(w.q), dev_u8(w.k), dev_u8(w.v), dev_i32(w.cu_seqlens_q),
                                   dev_i32(w.cu_seqlens_k), max(w.max_seqlen, 1),
                                   scale=float(w.scale), q_scale=float(w.q_scale),
                                   k_scale=float(w.k_scale), v_scale=float(w.v_scale),
                                   causal=causal)
    return host(o), host(lse)


def check_fp8(w, o, lse, causal):
    args = (w.cu_seqlens_q, w.cu_seqlens_k, w.scale, w.q_scale, w.k_scale, w.v_scale, causal)
    o_ref, lse_ref = oracle.attention_fp8_varlen(w.q, w.k, w.v, *args)
    o_abs, _ = oracle.attention_fp8_varlen(w.q, w.k, w.v & np.uint8(0x7F), *args)
    vmax = float(np.abs(oracle.e4m3_to_f64(w.v)).max()) * float(w.v_scale) if w.v.size else 0.0
    lk_row = np.zeros(o.shape[0])
    for s in range(len(w.lengths_q)):
        lk_row[w.cu_seqlens_q[s]:w.cu_seqlens_q[s + 1]] = w.lengths_k[s]
    bound = 2.0 ** -4 * o_abs + (2.0 ** -17 * lk_row * vmax)[:, None, None] + 1e-6
    err = np.abs(o.astype(np.float64) - o_ref)
    assert np.isfinite(o).all()
    worst = float((err / bound).max()) if err.size else 0.0
    assert worst <= 1.0, f"fp8 error exceeds its bound by {worst:.3f}x"
    check_lse(lse, lse_ref)
    rel = float(err.sum() / max(np.abs(o_ref).sum(), 1e-30))
    return {"max_err": float(err.max()) if err.size else 0.0, "worst_over_bound": worst,
            "sum_rel": rel}


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_fp8_varlen_ragged_gqa(d, causal):
    w = gen.make_fp8_varlen(f"f8v{d}", 2000 + d, [1, 7, 64, 100, 129, 300, 33], 4, 2, d, causal)
    o, lse = run_varlen(w)
    print(check_fp8(w, o, lse, causal))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_fp8_lq_ne_lk_and_empty(d, causal):
    w = gen.make_fp8_varlen("f8ne", 2100 + d, [5, 130, 0, 64, 3, 0], 2, 2, d, causal,
                            lengths_k=[9, 70, 12, 200, 0, 0])
    o, lse = run_varlen(w)
    print(check_fp8(w, o, lse, causal))


def test_fp8_factors():
    w = gen.make_fp8_varlen("f8fac", 2200, [77, 300], 4, 1, 128, True, factors=(0.5, 4.0, 0.125))
    o, lse = run_varlen(w)
    print(check_fp8(w, o, lse, True))


@pytest.mark.parametrize("causal", [True, False])
def test_fp8_dense_matches_varlen(causal):
    t = api()
    w = gen.make_fp8_varlen("f8d", 2300, [200, 200], 4, 2, 128, causal)
    o_v, l_v = run_varlen(w)
    q = dev_u8(w.q.reshape(2, 200, 4, 128))
    k = dev_u8(w.k.reshape(2, 200, 2, 128))
    v = dev_u8(w.v.reshape(2, 200, 2, 128))
    o_d, l_d = t.attn_fwd_fp8_dense(q, k, v, scale=float(w.scale), causal=causal)
    assert np.array_equal(host(o_d).reshape(o_v.shape), o_v)
    assert np.array_equal(host(l_d).transpose(1, 0, 2).reshape(l_v.shape), l_v)


def test_fp8_full_size_1x8192_sampled():
    """1 x 8192 causal, 16 heads, d=128: 64 sampled (query, head) rows against the oracle."""
    w = gen.make_fp8_varlen("f8big", 2400, [8192], 16, 16, 128, True)
    o, lse = run_varlen(w)
    r = np.random.Generator(np.random.PCG64(5))
    qd = oracle.e4m3_to_f64(w.q)
    kd = oracle.e4m3_to_f64(w.k)
    vd = oracle.e4m3_to_f64(w.v)
    for _ in range(64):
        i, h = int(r.integers(0, 8192)), int(r.integers(0, 16))
        o_ref, l_ref = oracle.attention_query(qd[i, h], kd[:, h], vd[:, h], w.scale, True, i, 8192)
        o_abs, _ = oracle.attention_query(qd[i, h], kd[:, h], np.abs(vd[:, h]), w.scale, True, i, 8192)
        bound = 2.0 ** -4 * o_abs + 2.0 ** -17 * 8192 * float(np.abs(vd).max()) + 1e-6
        assert (np.abs(o[i, h] - o_ref) <= bound).all(), (i, h)
        assert abs(lse[h, i] - l_ref) <= 1e-3
