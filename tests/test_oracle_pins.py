"""Pins for the fp64 oracle, independent of the oracle's own code.

The pages print no numeric attention outputs, so the oracle is pinned by
  * a brute-force per-query loop in pure Python (math.exp / math.fsum, no NumPy
    products) on tiny shapes;
  * closed forms: Q = 0 gives the mean of the visible V rows with
    LSE = ln(#visible); a dominant one-hot score (Hadamard keys) selects one V row;
  * invariants: probability rows sum to 1 with masked entries exactly 0, the
    causal prefix property, shift/affine/permutation invariances, and varlen
    packing equal to dense attention per sequence;
  * a hand-derived worked example stored under tests/golden/;
  * a library routine that is not the oracle's: torch's CPU float64
    scaled_dot_product_attention.
The mutation test at the end plants plausible mistakes in copies of the oracle
and checks that at least one pin rejects each.
"""

from __future__ import annotations

import json
import math
import os
import struct

import numpy as np
import pytest

import oracle
from oracle import attention as oatt
from synth import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------- helpers
def decode_bf16_struct(bits: np.ndarray) -> np.ndarray:
    """Independent bf16 decode: build each float32 from its bytes with struct."""
    flat = [struct.unpack("<f", struct.pack("<I", int(b) << 16))[0] for b in bits.reshape(-1)]
    return np.array(flat, dtype=np.float64).reshape(bits.shape)


def brute_attention(q, k, v, scale, causal):
    """Pure-Python per-query attention: lists and math only."""
    q = q.tolist()
    k = k.tolist()
    v = v.tolist()
    lq, lk, d = len(q), len(k), len(v[0]) if k else 0
    outs, lses = [], []
    for i in range(lq):
        vis = [j for j in range(lk) if (not causal) or j <= i + (lk - lq)]
        if not vis:
            outs.append([0.0] * len(q[i]))
            lses.append(-math.inf)
            continue
        sc = [scale * math.fsum(q[i][t] * k[j][t] for t in range(len(q[i]))) for j in vis]
        mx = max(sc)
        w = [math.exp(s - mx) for s in sc]
        tot = math.fsum(w)
        outs.append([math.fsum(w[n] * v[j][t] for n, j in enumerate(vis)) / tot for t in range(d)])
        lses.append(mx + math.log(tot))
    return np.array(outs), np.array(lses)


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def rand_f64(seed, *shape):
    return gen.bf16_bits_from_f32(rng(seed).standard_normal(size=shape, dtype=np.float32))


def assert_close(a, b, rtol=1e-12, atol=1e-12):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin)
    assert np.array_equal(a[~fin], b[~fin])
    np.testing.assert_allclose(a[fin], b[fin], rtol=rtol, atol=atol)


def hadamard(n):
    h = np.array([[1.0]])
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


# --------------------------------------------------------------------------- decode
def test_bf16_decode_matches_struct():
    bits = np.array([0x0000, 0x8000, 0x3F80, 0xBF80, 0x7F80, 0xFF80, 0x0001, 0x4049,
                     0x3EAA, 0x7F7F, 0xC2F7], dtype=np.uint16)
    got = oracle.bf16_bits_to_f64(bits)
    ref = decode_bf16_struct(bits)
    assert np.array_equal(got, ref)
    assert got[2] == 1.0 and got[3] == -1.0 and got[4] == math.inf
    assert got[7] == 3.140625
    assert math.copysign(1.0, got[1]) == -1.0


# --------------------------------------------------------------------------- brute force
BRUTE_CASES = [
    # (lq, lk, d, hq, hkv, causal)
    (7, 7, 32, 2, 2, False),
    (7, 7, 32, 2, 2, True),
    (5, 9, 64, 2, 1, True),     # Lq < Lk: bottom-right causal offset
    (9, 5, 64, 2, 1, True),     # Lq > Lk: first rows see nothing
    (6, 6, 128, 4, 2, True),    # GQA groups of 2
    (4, 11, 256, 1, 1, False),
    (1, 1, 32, 1, 1, True),
]


@pytest.mark.parametrize("lq,lk,d,hq,hkv,causal", BRUTE_CASES)
def test_dense_matches_brute_force(lq, lk, d, hq, hkv, causal):
    seed = 11 + lq * 7 + lk * 13 + d + causal
    qb = rand_f64(seed, 1, lq, hq, d)
    kb = rand_f64(seed + 1, 1, lk, hkv, d)
    vb = rand_f64(seed + 2, 1, lk, hkv, d)
    scale = np.float32(1.0 / math.sqrt(d))
    o, lse = oracle.attention_dense(qb, kb, vb, scale, causal)
    q, k, v = decode_bf16_struct(qb), decode_bf16_struct(kb), decode_bf16_struct(vb)
    for h in range(hq):
        g = h // (hq // hkv)
        bo, bl = brute_attention(q[0, :, h], k[0, :, g], v[0, :, g], float(scale), causal)
        assert_close(o[0, :, h], bo)
        assert_close(lse[0, h], bl)


def test_varlen_matches_brute_force_with_empty_sequence():
    lens_q = [3, 0, 8, 1]
    lens_k = [5, 2, 8, 4]
    d, hq, hkv = 32, 4, 2
    qb = rand_f64(21, sum(lens_q), hq, d)
    kb = rand_f64(22, sum(lens_k), hkv, d)
    vb = rand_f64(23, sum(lens_k), hkv, d)
    cq, ck = gen.cu_seqlens_from_lengths(lens_q), gen.cu_seqlens_from_lengths(lens_k)
    scale = np.float32(0.3)
    o, lse = oracle.attention_varlen(qb, kb, vb, cq, ck, scale, True)
    q, k, v = decode_bf16_struct(qb), decode_bf16_struct(kb), decode_bf16_struct(vb)
    for s in range(len(lens_q)):
        for h in range(hq):
            g = h // 2
            bo, bl = brute_attention(q[cq[s]:cq[s + 1], h], k[ck[s]:ck[s + 1], g],
                                     v[ck[s]:ck[s + 1], g], float(scale), True)
            if lens_q[s]:
                assert_close(o[cq[s]:cq[s + 1], h], bo)
                assert_close(lse[h, cq[s]:cq[s + 1]], bl)


NONPOS_CASES = [
    # (lq, lk, d, hq, hkv, causal, scale)
    (7, 7, 32, 2, 2, True, -0.25),
    (5, 9, 64, 2, 1, True, -0.125),
    (6, 6, 128, 4, 2, False, -1.0 / math.sqrt(128)),
    (6, 10, 64, 2, 2, True, 0.0),
    (4, 4, 32, 1, 1, False, 0.0),
]


@pytest.mark.parametrize("lq,lk,d,hq,hkv,causal,scale", NONPOS_CASES)
def test_nonpositive_scale_matches_brute_force(lq, lk, d, hq, hkv, causal, scale):
    """The definition holds for any finite scale: a negative one weights the
    smallest dot products highest, a zero one weights every visible key alike."""
    seed = 31 + lq * 5 + lk * 3 + d + causal
    qb = rand_f64(seed, 1, lq, hq, d)
    kb = rand_f64(seed + 1, 1, lk, hkv, d)
    vb = rand_f64(seed + 2, 1, lk, hkv, d)
    o, lse = oracle.attention_dense(qb, kb, vb, np.float32(scale), causal)
    q, k, v = decode_bf16_struct(qb), decode_bf16_struct(kb), decode_bf16_struct(vb)
    for h in range(hq):
        g = h // (hq // hkv)
        bo, bl = brute_attention(q[0, :, h], k[0, :, g], v[0, :, g], float(np.float32(scale)),
                                 causal)
        assert_close(o[0, :, h], bo)
        assert_close(lse[0, h], bl)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_scale_gives_mean_of_visible_values(causal):
    """Closed form: scale 0 makes every visible score 0 whatever Q and K hold."""
    lq, lk = 9, 13
    r = rng(61)
    q = r.standard_normal((lq, 32)) * 5.0
    k = r.standard_normal((lk, 32)) * 5.0
    v = r.standard_normal((lk, 32))
    o, lse = oracle.attention_one(q, k, v, 0.0, causal)
    for i in range(lq):
        n = i + 1 + (lk - lq) if causal else lk
        np.testing.assert_allclose(o[i], v[:n].mean(axis=0), rtol=0, atol=1e-13)
        assert abs(lse[i] - math.log(n)) < 1e-13


def test_negative_scale_selects_most_negative_dot_product():
    """Closed form: with Hadamard keys and q_i = -kappa H_t(i), a negative scale
    gives the single score -scale kappa^2 D at key t(i) and 0 elsewhere."""
    d, L, kappa = 64, 16, 3.0
    scale = -1.0 / math.sqrt(d)
    targets = [(5 * i + 2) % L for i in range(L)]
    q, k = _onehot_case(d, L, kappa, targets)
    q = -q
    v = rng(62).standard_normal((L, d))
    o, lse = oracle.attention_one(q, k, v, scale, False)
    delta = -scale * kappa * kappa * d
    for i in range(L):
        np.testing.assert_allclose(o[i], v[targets[i]], rtol=0, atol=L * math.exp(-delta) * 10)
        assert abs(lse[i] - (delta + math.log1p((L - 1) * math.exp(-delta)))) < 1e-12


# --------------------------------------------------------------------------- invariants
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("lq,lk", [(16, 16), (8, 20), (20, 8)])
def test_probability_rows_sum_to_one_and_masked_are_zero(causal, lq, lk):
    r = rng(5)
    q = r.standard_normal((lq, 32))
    k = r.standard_normal((lk, 32))
    p, m, l = oracle.softmax_probs(q, k, 0.7, causal)
    vis = np.array([[(not causal) or j <= i + lk - lq for j in range(lk)] for i in range(lq)])
    assert np.all(p[~vis] == 0.0)
    has = vis.any(axis=1)
    np.testing.assert_allclose(p[has].sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(p[~has] == 0.0)
    assert np.all(p >= 0.0)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_gives_mean_of_visible_values(causal):
    lq = lk = 12
    r = rng(6)
    q = np.zeros((lq, 64))
    k = r.standard_normal((lk, 64))
    v = r.standard_normal((lk, 64))
    o, lse = oracle.attention_one(q, k, v, 0.125, causal)
    for i in range(lq):
        n = i + 1 if causal else lk
        np.testing.assert_allclose(o[i], v[:n].mean(axis=0), rtol=0, atol=1e-13)
        assert abs(lse[i] - math.log(n)) < 1e-13


def _onehot_case(d, L, kappa, targets):
    h = hadamard(d)
    k = kappa * h[:L]
    q = kappa * h[np.asarray(targets)]
    return q, k


@pytest.mark.parametrize("d", [32, 64, 128])
def test_onehot_dominant_score_selects_value_row(d):
    L = min(d, 16)
    kappa = 3.0
    scale = 1.0 / math.sqrt(d)
    delta = scale * kappa * kappa * d
    assert delta >= 40
    targets = [(3 * i + 1) % L for i in range(L)]
    q, k = _onehot_case(d, L, kappa, targets)
    v = rng(7).standard_normal((L, d))
    o, lse = oracle.attention_one(q, k, v, scale, False)
    for i in range(L):
        np.testing.assert_allclose(o[i], v[targets[i]], rtol=0, atol=L * math.exp(-40) * 10)
        expect = delta + math.log1p((L - 1) * math.exp(-delta))
        assert abs(lse[i] - expect) < 1e-12


def test_onehot_future_target_is_masked_under_causal():
    # Each row's dominant key lies in its future; a correct causal mask leaves
    # only zero scores, i.e. the prefix mean with LSE = ln(i+1).
    d, L = 32, 16
    kappa = 3.0
    targets = [min(i + 1 + (i % 3), L - 1) for i in range(L - 1)]
    q, k = _onehot_case(d, L, kappa, targets)
    q = np.vstack([q, np.zeros((1, d))])      # last query: no future key exists; use Q = 0
    v = rng(8).standard_normal((L, d))
    o, lse = oracle.attention_one(q, k, v, 1.0 / math.sqrt(d), True)
    # without the mask each row would select its future target instead
    o_nc, _ = oracle.attention_one(q, k, v, 1.0 / math.sqrt(d), False)
    np.testing.assert_allclose(o_nc[:L - 1], v[targets], rtol=0, atol=1e-12)
    for i in range(L - 1):
        np.testing.assert_allclose(o[i], v[:i + 1].mean(axis=0), rtol=0, atol=1e-12)
        assert abs(lse[i] - math.log(i + 1)) < 1e-12


def test_causal_prefix_property_and_future_perturbation():
    L, d = 24, 32
    r = rng(9)
    q, k, v = (r.standard_normal((L, d)) for _ in range(3))
    o, lse = oracle.attention_one(q, k, v, 0.2, True)
    for i in range(L):
        oi, li = oracle.attention_one(q[i:i + 1], k[:i + 1], v[:i + 1], 0.2, False)
        np.testing.assert_allclose(o[i], oi[0], rtol=1e-13, atol=1e-14)
        assert abs(lse[i] - li[0]) < 1e-13
    k2, v2 = k.copy(), v.copy()
    k2[10:] += 5.0
    v2[10:] -= 3.0
    o2, lse2 = oracle.attention_one(q, k2, v2, 0.2, True)
    assert np.array_equal(o2[:10], o[:10]) and np.array_equal(lse2[:10], lse[:10])
    assert not np.allclose(o2[10:], o[10:])


def test_shift_and_affine_invariances():
    lq, lk, d = 10, 14, 64
    r = rng(10)
    q, k, v = r.standard_normal((lq, d)), r.standard_normal((lk, d)), r.standard_normal((lk, d))
    scale = 0.125
    o, lse = oracle.attention_one(q, k, v, scale, False)
    u = r.standard_normal(d)
    o_u, lse_u = oracle.attention_one(q, k + u, v, scale, False)
    np.testing.assert_allclose(o_u, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse_u, lse + scale * (q @ u), rtol=0, atol=1e-12)
    w = r.standard_normal(d)
    o_w, _ = oracle.attention_one(q, k, v + w, scale, False)
    np.testing.assert_allclose(o_w, o + w, rtol=0, atol=1e-12)
    perm = r.permutation(lk)
    o_p, lse_p = oracle.attention_one(q, k[perm], v[perm], scale, False)
    np.testing.assert_allclose(o_p, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse_p, lse, rtol=0, atol=1e-12)
    qperm = r.permutation(lq)
    o_q, lse_q = oracle.attention_one(q[qperm], k, v, scale, False)
    np.testing.assert_allclose(o_q, o[qperm], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse_q, lse[qperm], rtol=0, atol=1e-13)
    # scale acts on scores: doubling scale equals doubling q
    o_s, lse_s = oracle.attention_one(q, k, v, 2 * scale, False)
    o_2q, lse_2q = oracle.attention_one(2 * q, k, v, scale, False)
    np.testing.assert_allclose(o_s, o_2q, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse_s, lse_2q, rtol=0, atol=1e-12)


def test_varlen_equals_dense_per_sequence():
    lens = [5, 17, 1, 9]
    d, hq, hkv = 64, 4, 1
    w = gen.make_varlen("t", 31, lens, hq, hkv, d, True)
    o, lse = oracle.attention_varlen(w.q, w.k, w.v, w.cu_seqlens_q, w.cu_seqlens_k, w.scale, True)
    c = w.cu_seqlens_q
    for s, L in enumerate(lens):
        od, ld = oracle.attention_dense(w.q[None, c[s]:c[s + 1]], w.k[None, c[s]:c[s + 1]],
                                        w.v[None, c[s]:c[s + 1]], w.scale, True)
        assert np.array_equal(o[c[s]:c[s + 1]], od[0])
        assert np.array_equal(lse[:, c[s]:c[s + 1]], ld[0])


def test_attention_query_matches_full():
    w = gen.make_varlen("t", 41, [33, 12], 2, 2, 32, True, lengths_k=[40, 12])
    o, lse = oracle.attention_varlen(w.q, w.k, w.v, w.cu_seqlens_q, w.cu_seqlens_k, w.scale, True)
    q = oracle.bf16_bits_to_f64(w.q)
    k = oracle.bf16_bits_to_f64(w.k)
    v = oracle.bf16_bits_to_f64(w.v)
    for (s, i, h) in [(0, 0, 0), (0, 32, 1), (1, 5, 1), (1, 11, 0)]:
        q0, k0, k1 = w.cu_seqlens_q[s], w.cu_seqlens_k[s], w.cu_seqlens_k[s + 1]
        orow, l = oracle.attention_query(q[q0 + i, h], k[k0:k1, h], v[k0:k1, h], w.scale, True, i,
                                         w.lengths_q[s])
        np.testing.assert_allclose(orow, o[q0 + i, h], rtol=1e-12, atol=1e-13)
        assert abs(l - lse[h, q0 + i]) < 1e-12


def test_torch_sdpa_float64_agrees():
    torch = pytest.importorskip("torch")
    r = rng(12)
    for causal in (False, True):
        q, k, v = (r.standard_normal((2, 3, 20, 32)) for _ in range(3))
        o, lse = oracle.attention_dense(gen.bf16_bits_from_f32(q.transpose(0, 2, 1, 3).astype(np.float32)),
                                        gen.bf16_bits_from_f32(k.transpose(0, 2, 1, 3).astype(np.float32)),
                                        gen.bf16_bits_from_f32(v.transpose(0, 2, 1, 3).astype(np.float32)),
                                        np.float32(0.25), causal)
        dq = decode_bf16_struct(gen.bf16_bits_from_f32(q.astype(np.float32)))
        dk = decode_bf16_struct(gen.bf16_bits_from_f32(k.astype(np.float32)))
        dv = decode_bf16_struct(gen.bf16_bits_from_f32(v.astype(np.float32)))
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(dq), torch.from_numpy(dk), torch.from_numpy(dv),
            is_causal=causal, scale=0.25).numpy()
        np.testing.assert_allclose(o.transpose(0, 2, 1, 3), ref, rtol=1e-10, atol=1e-12)


def test_golden_worked_example():
    with open(os.path.join(GOLDEN, "attention_worked_example.json")) as f:
        ex = json.load(f)
    for case in ex["cases"]:
        o, lse = oracle.attention_one(np.array(case["q"], float), np.array(case["k"], float),
                                      np.array(case["v"], float), case["scale"], case["causal"])
        np.testing.assert_allclose(o, np.array(case["o"], float), rtol=0, atol=1e-12)
        exp_lse = [(-math.inf if x is None else x) for x in case["lse"]]
        assert_close(lse, np.array(exp_lse), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------- gather / scatter
def test_gather_scatter_golden_and_round_trip():
    with open(os.path.join(GOLDEN, "gather_scatter_example.json")) as f:
        ex = json.load(f)
    src = np.array(ex["padded"], dtype=np.uint16)
    idx = np.array(ex["indices"], dtype=np.int32)
    packed = oracle.unpad_gather(src, idx, src.shape[1:])
    assert np.array_equal(packed, np.array(ex["packed"], dtype=np.uint16))
    back = oracle.pad_scatter(packed, idx, src.shape[0])
    assert np.array_equal(back, np.array(ex["repadded"], dtype=np.uint16))


def test_gather_scatter_bytes_against_loop_and_nan_padding():
    w = gen.make_padded("t", 51, 64, [16, 16, 16], 2, 32, True, random_max=16, pad_value=float("nan"))
    raw = w.q.reshape(64, -1).view(np.uint8).reshape(64, -1)
    packed = oracle.unpad_gather(w.q, w.indices, w.q.shape[2:])
    pb = packed.reshape(len(w.indices), -1).view(np.uint8)
    for r, i in enumerate(w.indices):
        assert bytes(pb[r]) == bytes(raw[i])
    # no NaN-poisoned padding row reaches the packed tensor
    assert not np.isnan(oracle.bf16_bits_to_f64(packed)).any()
    back = oracle.pad_scatter(packed, w.indices, 64)
    valid = np.zeros(64, bool)
    valid[w.indices] = True
    assert np.array_equal(back[valid], w.q[0, valid])
    assert np.all(back[~valid] == 0)


# --------------------------------------------------------------------------- mutation test
def _mutants():
    """Copies of oracle.attention_one with one plausible mistake each."""
    def no_scale(q, k, v, scale, causal):
        return oatt.attention_one(q, k, v, 1.0, causal)

    def wrong_causal_offset(q, k, v, scale, causal):
        lq, lk = q.shape[0], k.shape[0]
        s = scale * (q @ k.T)
        vis = np.tril(np.ones((lq, lk), bool)) if causal else np.ones((lq, lk), bool)  # top-left
        s = np.where(vis, s, -np.inf)
        m = s.max(axis=1)
        e = np.exp(s - m[:, None])
        l = e.sum(axis=1)
        return (e @ v) / l[:, None], m + np.log(l)

    def strict_causal(q, k, v, scale, causal):
        lq, lk = q.shape[0], k.shape[0]
        s = scale * (q @ k.T)
        if causal:
            vis = np.arange(lk)[None, :] < np.arange(lq)[:, None] + (lk - lq)
            s = np.where(vis, s, -np.inf)
        m = s.max(axis=1)
        m = np.where(np.isfinite(m), m, 0)
        e = np.exp(s - m[:, None])
        l = e.sum(axis=1)
        return (e @ v) / np.maximum(l, 1e-300)[:, None], m + np.log(np.maximum(l, 1e-300))

    def lse_without_max(q, k, v, scale, causal):
        o, lse = oatt.attention_one(q, k, v, scale, causal)
        p, m, l = oatt.softmax_probs(q, k, scale, causal)
        return o, np.log(l)

    def transposed_v_use(q, k, v, scale, causal):
        p, m, l = oatt.softmax_probs(q, k, scale, causal)
        o = p @ v[::-1]
        return o, m + np.log(l)

    def unnormalised(q, k, v, scale, causal):
        p, m, l = oatt.softmax_probs(q, k, scale, causal)
        return (p * l[:, None]) @ v, m + np.log(l)

    def sign_flip(q, k, v, scale, causal):
        return oatt.attention_one(q, -k, v, scale, causal)

    return [no_scale, wrong_causal_offset, strict_causal, lse_without_max, transposed_v_use,
            unnormalised, sign_flip]


def _pins_pass(fn) -> bool:
    """Run a subset of the pins above against an attention_one-like function."""
    try:
        r = rng(99)
        # brute force, Lq < Lk causal, and non-causal
        for (lq, lk, causal) in [(5, 9, True), (6, 6, False), (6, 6, True)]:
            q, k, v = r.standard_normal((lq, 16)), r.standard_normal((lk, 16)), r.standard_normal((lk, 16))
            o, lse = fn(q, k, v, 0.3, causal)
            bo, bl = brute_attention(q, k, v, 0.3, causal)
            if not (np.allclose(o, bo, atol=1e-10) and np.allclose(lse, bl, atol=1e-10)):
                return False
        # Q = 0 closed form
        k, v = r.standard_normal((8, 16)), r.standard_normal((8, 16))
        o, lse = fn(np.zeros((8, 16)), k, v, 0.3, True)
        for i in range(8):
            if not (np.allclose(o[i], v[:i + 1].mean(0), atol=1e-12) and abs(lse[i] - math.log(i + 1)) < 1e-12):
                return False
        return True
    except Exception:
        return False


def test_pins_accept_oracle_and_reject_mutants():
    assert _pins_pass(oatt.attention_one)
    for m in _mutants():
        assert not _pins_pass(m), m.__name__


def test_gather_scatter_empty_index_list():
    src = np.arange(24, dtype=np.float32).reshape(6, 2, 2)
    g = oracle.unpad_gather(src, np.zeros(0, np.int32), (2, 2))
    assert g.shape == (0, 2, 2)
    s = oracle.pad_scatter(np.zeros((0, 2, 2), np.float32), np.zeros(0, np.int32), 5)
    assert s.shape == (5, 2, 2) and np.all(s == 0)
