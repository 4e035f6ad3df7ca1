"""CPU pins of the fp64 gradient oracle (oracle/backward.py).

Each pin is independent of the function under test: central finite
differences of the forward oracle, torch autograd in fp64 (a library
routine), exact identities that follow from the definition, and the sum over
the query heads of a grouped key/value head.  A mutation test checks that a
plausible mistake in the gradient code fails at least one pin.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from oracle import attention as oatt
from oracle import backward as obw
from synth import gen

CASES = [(5, 5, True), (4, 7, True), (7, 4, True), (6, 6, False), (3, 8, False)]


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _finite_difference_ok(fn, lq, lk, causal, seed, d=4, scale=0.45, eps=1e-6, tol=1e-7):
    r = rng(seed)
    q, k, v = r.standard_normal((lq, d)), r.standard_normal((lk, d)), r.standard_normal((lk, d))
    w = r.standard_normal((lq, d))  # upstream gradient dO

    def loss(qq, kk, vv):
        o, _ = oatt.attention_one(qq, kk, vv, scale, causal)
        return float((o * w).sum())

    dq, dk, dv = fn(q, k, v, w, scale, causal)
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            save = x[idx]
            x[idx] = save + eps
            lp = loss(q, k, v)
            x[idx] = save - eps
            lm = loss(q, k, v)
            x[idx] = save
            num[idx] = (lp - lm) / (2 * eps)
        if not np.allclose(num, g, atol=tol, rtol=1e-6):
            return False
    return True


@pytest.mark.parametrize("lq,lk,causal", CASES)
def test_gradient_matches_central_finite_differences(lq, lk, causal):
    assert _finite_difference_ok(obw.attention_backward_one, lq, lk, causal, seed=lq * 31 + lk)


def test_gradient_matches_torch_autograd_fp64():
    import torch
    r = rng(5)
    for lq, lk, causal in CASES:
        if causal and lq > lk:
            continue  # rows with no visible key: torch's softmax gives NaN (pinned separately)
        q, k, v = r.standard_normal((lq, 8)), r.standard_normal((lk, 8)), r.standard_normal((lk, 8))
        do = r.standard_normal((lq, 8))
        tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
        s = 0.3 * tq @ tk.T
        if causal:
            vis = torch.tensor(oatt.visible_mask(lq, lk, True))
            s = s.masked_fill(~vis, float("-inf"))
        o = torch.softmax(s, dim=-1) @ tv
        o.backward(torch.tensor(do))
        dq, dk, dv = obw.attention_backward_one(q, k, v, do, 0.3, causal)
        assert np.allclose(dq, tq.grad.numpy(), atol=1e-12)
        assert np.allclose(dk, tk.grad.numpy(), atol=1e-12)
        assert np.allclose(dv, tv.grad.numpy(), atol=1e-12)


def test_identities_from_the_definition():
    r = rng(11)
    lq, lk, d = 9, 9, 8
    q, k, v, do = (r.standard_normal((n, d)) for n in (lq, lk, lk, lq))
    for causal in (True, False):
        dq, dk, dv = obw.attention_backward_one(q, k, v, do, 0.5, causal)
        # every query row sees a key and its P row sums to 1: sum_j dV_j = sum_i dO_i
        assert np.allclose(dv.sum(axis=0), do.sum(axis=0), atol=1e-12)
        # rows of dS sum to 0, so sum_j dK_j = scale * sum_i Q_i * (sum_j dS_ij) = 0
        assert np.allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    # identical keys: P does not depend on q, so dQ = 0
    kk = np.tile(r.standard_normal((1, d)), (lk, 1))
    dq, _, _ = obw.attention_backward_one(q, kk, v, do, 0.5, True)
    assert np.allclose(dq, 0.0, atol=1e-12)


def test_masked_rows_and_fully_masked_queries():
    # Lq > Lk causal: the first queries see no key -> zero dq, no contribution
    r = rng(12)
    q, k, v, do = r.standard_normal((6, 4)), r.standard_normal((3, 4)), r.standard_normal((3, 4)), r.standard_normal((6, 4))
    dq, dk, dv = obw.attention_backward_one(q, k, v, do, 0.7, True)
    assert np.all(dq[:3] == 0)
    dq2, dk2, dv2 = obw.attention_backward_one(q[3:], k, v, do[3:], 0.7, True)
    assert np.allclose(dk, dk2, atol=1e-14) and np.allclose(dv, dv2, atol=1e-14)


def test_grouped_heads_sum_over_the_group():
    w = gen.make_varlen("bwgqa", 21, [7, 0, 5], 4, 2, 16, True)
    r = rng(13)
    do = gen.normal_bf16(r, w.q.shape)
    dq, dk, dv = oracle.attention_backward_varlen(w.q, w.k, w.v, do, w.cu_seqlens_q,
                                                  w.cu_seqlens_k, w.scale, True)
    # expand k/v to one head per query head and sum the per-head gradients
    k_rep = np.repeat(w.k, 2, axis=1)
    v_rep = np.repeat(w.v, 2, axis=1)
    dq2, dk2, dv2 = oracle.attention_backward_varlen(w.q, k_rep, v_rep, do, w.cu_seqlens_q,
                                                     w.cu_seqlens_k, w.scale, True)
    assert np.allclose(dq, dq2)
    assert np.allclose(dk, dk2.reshape(dk2.shape[0], 2, 2, -1).sum(axis=2))
    assert np.allclose(dv, dv2.reshape(dv2.shape[0], 2, 2, -1).sum(axis=2))


def test_dense_equals_varlen():
    r = rng(14)
    wd = gen.make_dense("bwd", 22, 2, 6, 9, 2, 1, 16, True)
    do = gen.normal_bf16(r, wd.q.shape)
    a = oracle.attention_backward_dense(wd.q, wd.k, wd.v, do, wd.scale, True)
    cu_q = gen.cu_seqlens_from_lengths([6, 6])
    cu_k = gen.cu_seqlens_from_lengths([9, 9])
    b = oracle.attention_backward_varlen(wd.q.reshape(12, 2, 16), wd.k.reshape(18, 1, 16),
                                         wd.v.reshape(18, 1, 16), do.reshape(12, 2, 16),
                                         cu_q, cu_k, wd.scale, True)
    assert np.allclose(a[0].reshape(12, 2, 16), b[0])
    assert np.allclose(a[1].reshape(18, 1, 16), b[1])
    assert np.allclose(a[2].reshape(18, 1, 16), b[2])


# --------------------------------------------------------------------------- mutation test
def _mutants():
    def no_dsum(q, k, v, do, scale, causal):
        p, _, _ = oatt.softmax_probs(q, k, scale, causal)
        ds = p * (do @ v.T)
        return scale * ds @ k, scale * ds.T @ q, p.T @ do

    def no_scale(q, k, v, do, scale, causal):
        dq, dk, dv = obw.attention_backward_one(q, k, v, do, scale, causal)
        return dq / scale, dk / scale, dv

    def transposed_dk(q, k, v, do, scale, causal):
        p, _, _ = oatt.softmax_probs(q, k, scale, causal)
        dp = do @ v.T
        ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
        return scale * ds @ k, scale * (ds @ k)[: k.shape[0]] if q.shape[0] >= k.shape[0] else scale * ds.T @ k, p.T @ do

    def dv_from_ds(q, k, v, do, scale, causal):
        dq, dk, dv = obw.attention_backward_one(q, k, v, do, scale, causal)
        p, _, _ = oatt.softmax_probs(q, k, scale, causal)
        dp = do @ v.T
        ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
        return dq, dk, ds.T @ do

    def mask_ignored(q, k, v, do, scale, causal):
        return obw.attention_backward_one(q, k, v, do, scale, False)

    def column_dsum(q, k, v, do, scale, causal):
        p, _, _ = oatt.softmax_probs(q, k, scale, causal)
        dp = do @ v.T
        ds = p * (dp - (p * dp).sum(axis=0, keepdims=True))
        return scale * ds @ k, scale * ds.T @ q, p.T @ do

    return [no_dsum, no_scale, transposed_dk, dv_from_ds, mask_ignored, column_dsum]


def _pins_pass(fn) -> bool:
    try:
        for lq, lk, causal in [(5, 5, True), (4, 6, True), (5, 5, False)]:
            if not _finite_difference_ok(fn, lq, lk, causal, seed=lq + 10 * lk):
                return False
        return True
    except Exception:
        return False


def test_pins_accept_oracle_and_reject_mutants():
    assert _pins_pass(obw.attention_backward_one)
    for m in _mutants():
        assert not _pins_pass(m), m.__name__
