"""fp64 reference attention -- TEST INFRASTRUCTURE ONLY (see the package docstring).

Written from the definition on the page "Intro to FlashAttention on Ascend
CANN" (section "where the traditional implementation is slow"): scores are
Q K^T scaled by 1/sqrt(d_k), a row softmax turns them into weights, and the
weights multiply V.  The full score matrix is materialised on purpose; no
tiling, no online rescaling, no reordering.

Readings where the pages are silent (each stated once here):
  * scale is an explicit float32 argument (the pages use 1/sqrt(d_k)); it is
    widened to fp64 unchanged.
  * causal masking aligns bottom-right: key j is visible to query i when
    j <= i + (Lk - Lq); with Lq == Lk this is the usual j <= i.
  * LSE is the natural-log log-sum-exp of the scaled visible scores of a row.
  * a row with no visible key has output 0 and LSE -inf.
  * grouped-query heads: query head h reads key/value head h // (Hq // Hkv).
"""

from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact decode of bfloat16 bit patterns (uint16) to float64."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def visible_mask(lq: int, lk: int, causal: bool) -> np.ndarray:
    """Boolean (lq, lk) matrix: True where query i may attend to key j."""
    if not causal:
        return np.ones((lq, lk), dtype=bool)
    i = np.arange(lq)[:, None]
    j = np.arange(lk)[None, :]
    return j <= i + (lk - lq)


def softmax_probs(q: np.ndarray, k: np.ndarray, scale: float, causal: bool):
    """Row-softmax weights of the scaled scores, with masked entries exactly 0.

    q: (Lq, D) float64, k: (Lk, D) float64.  Returns (P, m, l) where P is
    (Lq, Lk), m the row maximum of the visible scaled scores and l the row sum
    of exp(score - m).  Rows with no visible key have P = 0, m = -inf, l = 0.
    """
    lq, lk = q.shape[0], k.shape[0]
    s = float(scale) * (q @ k.T)                      # full (Lq, Lk) score matrix
    vis = visible_mask(lq, lk, causal)
    s_vis = np.where(vis, s, -np.inf)
    m = s_vis.max(axis=1) if lk > 0 else np.full(lq, -np.inf)
    has_key = np.isfinite(m)
    m_safe = np.where(has_key, m, 0.0)
    e = np.where(vis, np.exp(s_vis - m_safe[:, None]), 0.0)
    l = e.sum(axis=1)
    p = np.zeros_like(e)
    p[has_key] = e[has_key] / l[has_key, None]
    return p, m, l


def attention_one(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, causal: bool):
    """Attention for one (sequence, head): q (Lq, D), k/v (Lk, D) float64.

    Returns O (Lq, D) float64 and LSE (Lq,) float64.
    """
    p, m, l = softmax_probs(q, k, scale, causal)
    o = p @ v
    with np.errstate(divide="ignore"):
        lse = np.where(np.isfinite(m), m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return o, lse


def attention_dense(q_bits, k_bits, v_bits, scale, causal: bool):
    """Dense batched attention on bfloat16 bit patterns.

    q (B, Sq, Hq, D), k/v (B, Sk, Hkv, D) uint16.  Returns O (B, Sq, Hq, D)
    float64 and LSE (B, Hq, Sq) float64.
    """
    q = bf16_bits_to_f64(q_bits)
    k = bf16_bits_to_f64(k_bits)
    v = bf16_bits_to_f64(v_bits)
    b, sq, hq, d = q.shape
    hkv = k.shape[2]
    group = hq // hkv
    o = np.zeros((b, sq, hq, d))
    lse = np.zeros((b, hq, sq))
    for bi in range(b):
        for h in range(hq):
            g = h // group
            o[bi, :, h, :], lse[bi, h, :] = attention_one(
                q[bi, :, h, :], k[bi, :, g, :], v[bi, :, g, :], np.float32(scale), causal)
    return o, lse


def attention_varlen(q_bits, k_bits, v_bits, cu_seqlens_q, cu_seqlens_k, scale, causal: bool):
    """Variable-length packed attention on bfloat16 bit patterns.

    q (Tq, Hq, D), k/v (Tk, Hkv, D) uint16; sequence s owns query rows
    cu_seqlens_q[s]:cu_seqlens_q[s+1] and key rows cu_seqlens_k[s]:cu_seqlens_k[s+1].
    Returns O (Tq, Hq, D) float64 and LSE (Hq, Tq) float64.
    """
    q = bf16_bits_to_f64(q_bits)
    k = bf16_bits_to_f64(k_bits)
    v = bf16_bits_to_f64(v_bits)
    tq, hq, d = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    o = np.zeros((tq, hq, d))
    lse = np.full((hq, tq), -np.inf)
    cq = np.asarray(cu_seqlens_q, dtype=np.int64)
    ck = np.asarray(cu_seqlens_k, dtype=np.int64)
    for s in range(len(cq) - 1):
        q0, q1, k0, k1 = cq[s], cq[s + 1], ck[s], ck[s + 1]
        if q1 == q0:
            continue
        for h in range(hq):
            g = h // group
            o[q0:q1, h, :], lse[h, q0:q1] = attention_one(
                q[q0:q1, h, :], k[k0:k1, g, :], v[k0:k1, g, :], np.float32(scale), causal)
    return o, lse


def attention_query(q_row, k_seq, v_seq, scale, causal: bool, i: int, lq: int):
    """One query row of one (sequence, head), for sampled checks at full size.

    q_row (D,) float64 is query i of a sequence of lq queries; k_seq/v_seq
    (Lk, D) float64 are that sequence's keys and values.  Returns (O row, LSE).
    """
    lk = k_seq.shape[0]
    limit = lk if not causal else min(lk, i + (lk - lq) + 1)
    if limit <= 0:
        return np.zeros(q_row.shape[0]), -np.inf
    s = float(np.float32(scale)) * (k_seq[:limit] @ q_row)
    m = s.max()
    e = np.exp(s - m)
    l = e.sum()
    return (e @ v_seq[:limit]) / l, m + np.log(l)
