"""fp64 reference for attention on fp8 inputs -- TEST INFRASTRUCTURE ONLY.

The pages point to FP8 only in passing: Lesson 5 closes by pointing back to
FA-3's FP8 path, and "why FA is 2x on A100 but 1.5x on Ascend 910" (section 5)
recommends narrower KV data (INT8 KV) to halve the bytes moved.  Neither page
fixes a format.  The plainest reading, followed here: q, k and v are stored as
8-bit floats in the OCP E4M3 format (1 sign bit, 4 exponent bits with bias 7,
3 mantissa bits; exponent field 0 encodes subnormals, the all-ones pattern
S.1111.111 is NaN, there are no infinities), each tensor with one float32
dequantisation factor (value = decoded byte * factor).  The attention is the
standard definition (attention.py) on the dequantised values; nothing about the
kernel's own rounding (for instance of the probabilities) enters here.
"""

from __future__ import annotations

import numpy as np

from .attention import attention_one


def _e4m3_table() -> np.ndarray:
    t = np.empty(256, dtype=np.float64)
    for b in range(256):
        sign = -1.0 if b & 0x80 else 1.0
        e = (b >> 3) & 0xF
        m = b & 0x7
        if e == 0xF and m == 0x7:
            t[b] = np.nan
        elif e == 0:
            t[b] = sign * (m / 8.0) * 2.0 ** (1 - 7)
        else:
            t[b] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


E4M3 = _e4m3_table()


def e4m3_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode E4M3 bytes (uint8 array) to float64."""
    return E4M3[np.asarray(bits, dtype=np.uint8)]


def attention_fp8_varlen(q8, k8, v8, cu_seqlens_q, cu_seqlens_k, scale, q_scale, k_scale, v_scale,
                         causal: bool):
    """q8 (Tq, Hq, D), k8 / v8 (Tk, Hkv, D) E4M3 bytes; per-tensor factors.
    Returns O (Tq, Hq, D) float64 and LSE (Hq, Tq) float64 (natural log of the
    scaled visible scores, as in attention.py)."""
    q = e4m3_to_f64(q8) * float(np.float32(q_scale))
    k = e4m3_to_f64(k8) * float(np.float32(k_scale))
    v = e4m3_to_f64(v8) * float(np.float32(v_scale))
    tq, hq, d = q.shape
    group = hq // k.shape[1]
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
            o[q0:q1, h], lse[h, q0:q1] = attention_one(q[q0:q1, h], k[k0:k1, g], v[k0:k1, g],
                                                       np.float32(scale), causal)
    return o, lse


def attention_fp8_dense(q8, k8, v8, scale, q_scale, k_scale, v_scale, causal: bool):
    """Dense layout: q8 (B, Sq, Hq, D), k8 / v8 (B, Sk, Hkv, D).  Returns O
    (B, Sq, Hq, D) and LSE (B, Hq, Sq)."""
    b, sq = q8.shape[:2]
    sk = k8.shape[1]
    cu_q = np.arange(b + 1) * sq
    cu_k = np.arange(b + 1) * sk
    o, lse = attention_fp8_varlen(q8.reshape(b * sq, *q8.shape[2:]), k8.reshape(b * sk, *k8.shape[2:]),
                                  v8.reshape(b * sk, *v8.shape[2:]), cu_q, cu_k, scale, q_scale,
                                  k_scale, v_scale, causal)
    hq = q8.shape[2]
    return o.reshape(q8.shape), lse.reshape(hq, b, sq).transpose(1, 0, 2)
