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

import os

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


# Query blocks of the fp8 kernel: 128 (4 waves, 64-key tiles; the default) and
# 256 (8 waves, 128-key tiles); ATTN_FP8_TILE forces one.
@pytest.fixture(params=["128", "256"])
def fp8_tile(request, monkeypatch):
    monkeypatch.setenv("ATTN_FP8_TILE", request.param)
    return request.param


def run_checked(w, fp8_tile, causal):
    """run_varlen, except that head_dim 256 has 128-query blocks only: a forced
    256-query block must be refused before anything is launched."""
    if w.d == 256 and fp8_tile == "256":
        with pytest.raises(api().AttnError, match="UNSUPPORTED"):
            run_varlen(w)
        return None
    o, lse = run_varlen(w)
    return check_fp8(w, o, lse, causal)


@pytest.mark.parametrize("d", [32, 64, 128, 256])
@pytest.mark.parametrize("causal", [True, False])
def test_fp8_varlen_ragged_gqa(d, causal, fp8_tile):
    w = gen.make_fp8_varlen(f"f8v{d}", 2000 + d, [1, 7, 64, 100, 129, 300, 33, 700], 4, 2, d,
                            causal)
    print(run_checked(w, fp8_tile, causal))


@pytest.mark.parametrize("d", [32, 64, 128, 256])
@pytest.mark.parametrize("causal", [True, False])
def test_fp8_lq_ne_lk_and_empty(d, causal, fp8_tile):
    w = gen.make_fp8_varlen("f8ne", 2100 + d, [5, 130, 0, 64, 3, 0, 300], 2, 2, d, causal,
                            lengths_k=[9, 70, 12, 200, 0, 0, 190])
    print(run_checked(w, fp8_tile, causal))


@pytest.mark.parametrize("causal", [True, False])
def test_fp8_row_maximum_climbing_past_the_lift_range(causal, fp8_tile):
    """Q = 1.0 and keys whose magnitude doubles along the sequence (E4M3
    2^-6 .. 2^4, positive): a row's maximum climbs from ~0.3 to ~260 binades,
    in steps past the 32 binades that the PV product's operand scale carries,
    so the output rescale path runs as well as the lifted one."""
    w = gen.make_fp8_varlen("f8climb", 2300, [300, 129, 64], 2, 2, 128, causal)
    q = np.full_like(w.q, 0x38)  # 1.0
    k = w.k.copy()
    for s in range(len(w.lengths_k)):
        k0, k1 = int(w.cu_seqlens_k[s]), int(w.cu_seqlens_k[s + 1])
        e = 1 + (np.arange(k1 - k0) * 11) // max(k1 - k0, 1)  # exponent field 1..11
        k[k0:k1] = (e.astype(np.uint8) << 3)[:, None, None]
    w.q, w.k = q, k
    print(run_checked(w, fp8_tile, causal))


def test_fp8_factors(fp8_tile):
    w = gen.make_fp8_varlen("f8fac", 2200, [77, 300], 4, 1, 128, True, factors=(0.5, 4.0, 0.125))
    o, lse = run_varlen(w)
    print(check_fp8(w, o, lse, True))


@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("causal", [True, False])
def test_fp8_dense_matches_varlen(d, causal, fp8_tile):
    t = api()
    if d == 256 and fp8_tile == "256":
        pytest.skip("head_dim 256 has 128-query blocks only (the refusal is tested above)")
    w = gen.make_fp8_varlen("f8d", 2300 + d, [200, 200], 4, 2, d, causal)
    o_v, l_v = run_varlen(w)
    q = dev_u8(w.q.reshape(2, 200, 4, d))
    k = dev_u8(w.k.reshape(2, 200, 2, d))
    v = dev_u8(w.v.reshape(2, 200, 2, d))
    o_d, l_d = t.attn_fwd_fp8_dense(q, k, v, scale=float(w.scale), causal=causal)
    assert np.array_equal(host(o_d).reshape(o_v.shape), o_v)
    assert np.array_equal(host(l_d).transpose(1, 0, 2).reshape(l_v.shape), l_v)


@pytest.mark.parametrize("tile", [None, "256"])
def test_fp8_full_size_1x8192_whole_output(tile, monkeypatch):
    """1 x 8192 causal, 16 heads, d=128 (the fp8 benchmark shape; the default
    query block and the 256-query one): every output element within its bound,
    every LSE within 1e-3.  The oracle runs per head and per 1024-row block
    with the key prefix those rows see (the causal prefix property)."""
    w = gen.make_fp8_varlen("f8big", 2400, [8192], 16, 16, 128, True)
    if tile is None:
        assert "ATTN_FP8_TILE" not in os.environ
    else:
        monkeypatch.setenv("ATTN_FP8_TILE", tile)
    o, lse = run_varlen(w)
    assert np.isfinite(o).all()
    qd = oracle.e4m3_to_f64(w.q)
    kd = oracle.e4m3_to_f64(w.k)
    vd = oracle.e4m3_to_f64(w.v)
    vmax = float(np.abs(vd).max())
    scale = np.float32(w.scale)

    def one(h):
        worst, lerr = 0.0, 0.0
        for r0 in range(0, 8192, 1024):
            r1 = r0 + 1024
            o_ref, l_ref = oracle.attention_one(qd[r0:r1, h], kd[:r1, h], vd[:r1, h], scale, True)
            o_abs, _ = oracle.attention_one(qd[r0:r1, h], kd[:r1, h], np.abs(vd[:r1, h]), scale, True)
            bound = 2.0 ** -4 * o_abs + 2.0 ** -17 * 8192 * vmax + 1e-6
            worst = max(worst, float((np.abs(o[r0:r1, h] - o_ref) / bound).max()))
            lerr = max(lerr, float(np.abs(lse[h, r0:r1] - l_ref).max()))
        return worst, lerr

    import concurrent.futures
    with concurrent.futures.ThreadPoolExecutor(8) as ex:
        res = list(ex.map(one, range(16)))
    worst = max(r[0] for r in res)
    lerr = max(r[1] for r in res)
    print("fp8 1x8192: worst error / bound", worst, "max |dLSE|", lerr)
    assert worst <= 1.0 and lerr <= 1e-3
