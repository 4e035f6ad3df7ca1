"""GPU parity at full size: every element of the output of the large workloads.

The workloads are the dense ViT batch (149 x 12 heads, S=1024, d=64), the four
head_dim cases at S=4096, the 1 x 8192 varlen sequence, the 64/8-head GQA
sequence of 8192 and the 64K-token pack.  The GPU runs each workload once, in
the launch configuration the benchmark times (default tile policy, no split
workspace), and every (sequence, head) of its output is compared with the fp64
oracle: max |O - O_ref| <= 2e-2 and mean |O - O_ref| <= 2e-3 over all
elements, |LSE - LSE_ref| <= 1e-3 over all rows.

The oracle runs per (sequence, head) and, causal, per block of query rows with
the key prefix those rows can see: under the bottom-right rule of
oracle.attention_one, rows [r0, r1) against keys [0, r1 + Lk - Lq) are exactly
rows r0..r1-1 of the whole sequence (the causal prefix property that the
oracle's CPU pins check).  Each test covers a slice of the heads (or batches)
so that no single test runs for long; each slice must meet the mean bar on its
own, which implies it for the whole output.

Basis of the comparison: the tiled result equals the standard softmax
(page "Intro to FlashAttention on Ascend CANN", section "the first pitfall").
"""

from __future__ import annotations

import concurrent.futures
import os

import numpy as np
import pytest

import oracle
from synth import gen
from tests.gpu_util import LSE_MAX_ABS, O_MAX_ABS, O_MEAN_ABS, dev_bf16, dev_i32, host

pytestmark = pytest.mark.gpu

ROW_CHUNK = 1024


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


_CACHE: dict = {}


def _gpu_run(name: str):
    """(workload, O, LSE) of one full-size workload on the GPU, computed once
    per workload (the previous workload's arrays are dropped)."""
    if name in _CACHE:
        return _CACHE[name]
    _CACHE.clear()
    import tiled_attention_fwd_amd as t
    w = gen.build_workload(name)
    print(f"[fullsize] {name}: GPU run", flush=True)
    if w.kind == "dense":
        o, lse = t.attn_fwd_dense(dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v),
                                  scale=float(w.scale), causal=w.causal)
    else:
        o, lse = t.attn_fwd_varlen(dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v),
                                   dev_i32(w.cu_seqlens_q), dev_i32(w.cu_seqlens_k),
                                   w.max_seqlen, scale=float(w.scale), causal=w.causal)
    _CACHE[name] = (w, host(o), host(lse))
    return _CACHE[name]


def _compare_unit(o_g, l_g, qb, kb, vb, scale, causal):
    """One (sequence, head): GPU O (Lq, D) and LSE (Lq,) against the oracle.

    qb/kb/vb are bf16 bit patterns (Lq, D) / (Lk, D).  Returns (sum |dO|,
    max |dO|, element count, max |dLSE|)."""
    q = oracle.bf16_bits_to_f64(qb)
    k = oracle.bf16_bits_to_f64(kb)
    v = oracle.bf16_bits_to_f64(vb)
    lq, lk = q.shape[0], k.shape[0]
    if np.isnan(o_g).any() or np.isnan(l_g).any():
        return float("nan"), float("nan"), o_g.size, float("nan")
    s_err, m_err, l_err = 0.0, 0.0, 0.0
    for r0 in range(0, lq, ROW_CHUNK if causal else lq):
        r1 = min(lq, r0 + (ROW_CHUNK if causal else lq))
        kend = min(lk, r1 + lk - lq) if causal else lk
        kend = max(kend, 0)
        o_ref, lse_ref = oracle.attention_one(q[r0:r1], k[:kend], v[:kend], scale, causal)
        e = np.abs(o_g[r0:r1].astype(np.float64) - o_ref)
        s_err += float(e.sum())
        m_err = max(m_err, float(e.max()))
        fin = np.isfinite(lse_ref)
        lg = l_g[r0:r1]
        if not np.array_equal(np.isfinite(lg), fin):
            return float("nan"), float("nan"), o_g.size, float("nan")
        if fin.any():
            l_err = max(l_err, float(np.abs(lg[fin].astype(np.float64) - lse_ref[fin]).max()))
    return s_err, m_err, o_g.size, l_err


def _units(w, o, lse, part, n_parts):
    """(o, lse, q, k, v) slices of the (sequence, head) pairs of one part.
    Parts split the heads (several sequences: the sequences, for the ViT
    batch)."""
    group = w.hq // w.hkv
    if w.kind == "dense":
        b = w.q.shape[0]
        if b > 1:
            seqs = [s for s in range(b) if s % n_parts == part]
            heads = range(w.hq)
        else:
            seqs = [0]
            heads = [h for h in range(w.hq) if h * n_parts // w.hq == part]
        for s in seqs:
            for h in heads:
                g = h // group
                yield (o[s, :, h], lse[s, h], w.q[s, :, h], w.k[s, :, g], w.v[s, :, g])
    else:
        heads = [h for h in range(w.hq) if h * n_parts // w.hq == part]
        cq, ck = w.cu_seqlens_q, w.cu_seqlens_k
        for s in range(len(cq) - 1):
            q0, q1, k0, k1 = int(cq[s]), int(cq[s + 1]), int(ck[s]), int(ck[s + 1])
            if q1 == q0:
                continue
            for h in heads:
                g = h // group
                yield (o[q0:q1, h], lse[h, q0:q1], w.q[q0:q1, h], w.k[k0:k1, g], w.v[k0:k1, g])


# (workload, number of parts): a part is at most ~25 s of oracle time on 8
# host cores.  GQA: a part is one KV group (8 query heads).
CASES = [("vit_dense_b149", 4), ("hdim_sweep_d32", 2), ("hdim_sweep_d64", 1),
         ("hdim_sweep_d128", 1), ("hdim_sweep_d256", 1), ("varlen_1x8192", 1),
         ("gqa_dense_s8192", 8), ("pack_64k", 4)]
PARAMS = [(n, p, k) for n, k in CASES for p in range(k)]


@pytest.mark.parametrize("name,part,n_parts", PARAMS,
                         ids=[f"{n}-{p + 1}of{k}" for n, p, k in PARAMS])
def test_full_size_whole_output(name, part, n_parts):
    w, o, lse = _gpu_run(name)
    assert not np.isnan(o).any(), "NaN in GPU output"
    scale = np.float32(w.scale)
    units = list(_units(w, o, lse, part, n_parts))
    assert units
    with concurrent.futures.ThreadPoolExecutor(_workers()) as ex:
        res = list(ex.map(lambda u: _compare_unit(*u, scale, w.causal), units))
    assert not any(np.isnan(r[1]) for r in res), "NaN or finiteness mismatch in a unit"
    s_err = sum(r[0] for r in res)
    m_err = max(r[1] for r in res)
    n = sum(r[2] for r in res)
    l_err = max(r[3] for r in res)
    mean = s_err / n
    print(f"[fullsize] {name} part {part + 1}/{n_parts}: {len(units)} (sequence, head) pairs, "
          f"{n} elements, max {m_err:.3e}, mean {mean:.3e}, lse {l_err:.3e}", flush=True)
    assert m_err <= O_MAX_ABS, f"max abs err {m_err:.3e}"
    assert mean <= O_MEAN_ABS, f"mean abs err {mean:.3e}"
    assert l_err <= LSE_MAX_ABS, f"LSE err {l_err:.3e}"
