"""fp64 reference gradients of attention -- TEST INFRASTRUCTURE ONLY.

Gradient of the attention defined in attention.py with respect to q, k and v,
given the upstream gradient dO of the output.  The page "Intro to
FlashAttention on Ascend CANN" (section on the second pitfall, backward
propagation) says the backward pass recomputes the forward instead of keeping
the score matrix; the pages give no gradient formulas, so the plainest reading
is the exact derivative of the definition, written out with the chain rule:

  S = scale Q K^T,  P = softmax over the visible keys of each row,  O = P V
  dV = P^T dO
  dP = dO V^T
  dS = P * (dP - rowsum(P * dP))          (row softmax Jacobian)
  dQ = scale dS K
  dK = scale dS^T Q

Masked entries have P = 0, so their dS is 0; a row with no visible key
contributes nothing.  Grouped-query heads: the gradient of a key/value head is
the sum over the query heads that read it.  The full matrices are materialised
on purpose (no tiling, no recomputation order).
"""

from __future__ import annotations

import numpy as np

from .attention import bf16_bits_to_f64, softmax_probs


def attention_backward_one(q, k, v, do, scale, causal: bool):
    """One (sequence, query head): q (Lq, D), k, v (Lk, D), do (Lq, D), all
    float64.  Returns (dq (Lq, D), dk (Lk, D), dv (Lk, D))."""
    p, _, _ = softmax_probs(q, k, scale, causal)
    dv = p.T @ do
    dp = do @ v.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    dq = float(scale) * (ds @ k)
    dk = float(scale) * (ds.T @ q)
    return dq, dk, dv


def _heads_backward(qs, ks, vs, dos, scale, causal):
    """qs, dos (Lq, Hq, D); ks, vs (Lk, Hkv, D) float64 -> dq, dk, dv."""
    hq, hkv = qs.shape[1], ks.shape[1]
    group = hq // hkv
    dq = np.zeros_like(qs)
    dk = np.zeros_like(ks)
    dv = np.zeros_like(vs)
    for h in range(hq):
        g = h // group
        a, b, c = attention_backward_one(qs[:, h], ks[:, g], vs[:, g], dos[:, h], scale, causal)
        dq[:, h] = a
        dk[:, g] += b
        dv[:, g] += c
    return dq, dk, dv


def attention_backward_varlen(q_bits, k_bits, v_bits, do_bits, cu_seqlens_q, cu_seqlens_k,
                              scale, causal: bool):
    """Packed layout: q, do (Tq, Hq, D), k, v (Tk, Hkv, D) bf16 bit patterns.
    Returns float64 (dq, dk, dv) shaped like q, k, v."""
    q = bf16_bits_to_f64(q_bits)
    k = bf16_bits_to_f64(k_bits)
    v = bf16_bits_to_f64(v_bits)
    do = bf16_bits_to_f64(do_bits)
    scale = float(np.float32(scale))
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for s in range(len(cu_seqlens_q) - 1):
        q0, q1 = int(cu_seqlens_q[s]), int(cu_seqlens_q[s + 1])
        k0, k1 = int(cu_seqlens_k[s]), int(cu_seqlens_k[s + 1])
        a, b, c = _heads_backward(q[q0:q1], k[k0:k1], v[k0:k1], do[q0:q1], scale, causal)
        dq[q0:q1] = a
        dk[k0:k1] = b
        dv[k0:k1] = c
    return dq, dk, dv


def attention_backward_dense(q_bits, k_bits, v_bits, do_bits, scale, causal: bool):
    """Dense layout: q, do (B, Sq, Hq, D), k, v (B, Sk, Hkv, D) bf16 bit patterns."""
    q = bf16_bits_to_f64(q_bits)
    k = bf16_bits_to_f64(k_bits)
    v = bf16_bits_to_f64(v_bits)
    do = bf16_bits_to_f64(do_bits)
    scale = float(np.float32(scale))
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(q.shape[0]):
        dq[b], dk[b], dv[b] = _heads_backward(q[b], k[b], v[b], do[b], scale, causal)
    return dq, dk, dv
