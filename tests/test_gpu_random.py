"""Randomised GPU parity sweep (seeded): many small shapes through the default
tile policies and the fused padded path, each against the fp64 oracle.

Shapes are drawn so that every case stays small enough for the oracle while
still covering ragged tails, empty and single-row sequences, Lq != Lk per
sequence (bottom-right causal alignment), grouped heads and every head_dim.
"""

from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
from synth import gen
from tests.gpu_util import check_lse, check_o, dev_bf16, dev_i32, host

pytestmark = pytest.mark.gpu

N_CASES = 24


def api():
    import tiled_attention_fwd_amd as t
    return t


def _case(seed):
    r = np.random.Generator(np.random.PCG64(seed))
    d = int(r.choice([32, 64, 128, 256]))
    hkv = int(r.choice([1, 2, 3]))
    hq = hkv * int(r.choice([1, 2, 4]))
    nseq = int(r.integers(1, 6))
    kinds = r.integers(0, 4, size=nseq)
    lq, lk = [], []
    for kd in kinds:
        if kd == 0:
            a = int(r.integers(0, 3))            # empty or tiny
        else:
            a = int(r.integers(1, 400))
        b = a if r.random() < 0.6 else int(r.integers(0, 450))
        lq.append(a)
        lk.append(b)
    causal = bool(r.random() < 0.6)
    return d, hq, hkv, lq, lk, causal


@pytest.mark.parametrize("seed", range(7000, 7000 + N_CASES))
def test_random_varlen_vs_oracle(seed):
    t = api()
    d, hq, hkv, lq, lk, causal = _case(seed)
    if sum(lq) == 0:
        lq[0] = 1
    w = gen.make_varlen(f"rnd{seed}", seed, lq, hq, hkv, d, causal, lengths_k=lk)
    want_lse = seed % 3 != 0
    o, lse = t.attn_fwd_varlen(dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v),
                               dev_i32(w.cu_seqlens_q), dev_i32(w.cu_seqlens_k), max(lq),
                               scale=float(w.scale), causal=causal, return_lse=want_lse)
    o_ref, lse_ref = oracle.attention_varlen(w.q, w.k, w.v, w.cu_seqlens_q, w.cu_seqlens_k,
                                             w.scale, causal)
    check_o(host(o), o_ref)
    if want_lse:
        check_lse(host(lse), lse_ref)


@pytest.mark.parametrize("seed", range(7100, 7100 + 8))
def test_random_fused_padded_vs_oracle(seed):
    """Random right-padded slots (some empty) in a (B, total_len) layout."""
    t = api()
    r = np.random.Generator(np.random.PCG64(seed))
    d = int(r.choice([64, 128]))
    hkv = int(r.choice([1, 2]))
    hq = hkv * int(r.choice([1, 2]))
    b = int(r.integers(1, 3))
    total = int(r.choice([256, 384]))
    rows = b * total
    mask = np.zeros(rows, bool)
    pos = 0
    while pos < rows:
        slot = int(r.integers(16, 200))
        n = int(r.integers(0, slot + 1))
        mask[pos:min(rows, pos + n)] = True
        pos += slot
    if not mask.any():
        mask[0] = True
    # the sequences are the maximal runs of consecutive valid rows
    edges = np.diff(np.concatenate([[0], mask.astype(np.int8), [0]]))
    starts, ends = np.flatnonzero(edges == 1), np.flatnonzero(edges == -1)
    lens = [int(e - s) for s, e in zip(starts, ends)]
    idx = np.flatnonzero(mask).astype(np.int32)
    assert sum(lens) == len(idx)
    cu = gen.cu_seqlens_from_lengths(lens)
    q = gen.normal_bf16(r, (b, total, hq, d))
    k = gen.normal_bf16(r, (b, total, hkv, d))
    v = gen.normal_bf16(r, (b, total, hkv, d))
    causal = bool(seed % 2)
    out, lse = t.attn_fwd_padded(dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_i32(idx), dev_i32(cu),
                                 max(lens), causal=causal)
    out = host(out).reshape(rows, hq, d)
    gq = oracle.unpad_gather(q.reshape(rows, hq, d), idx, (hq, d))
    gk = oracle.unpad_gather(k.reshape(rows, hkv, d), idx, (hkv, d))
    gv = oracle.unpad_gather(v.reshape(rows, hkv, d), idx, (hkv, d))
    o_ref, lse_ref = oracle.attention_varlen(gq, gk, gv, cu, cu, np.float32(1 / math.sqrt(d)), causal)
    check_o(out, oracle.pad_scatter(o_ref, idx, rows))
    check_lse(host(lse), lse_ref)
    assert np.all(out[~mask].view(np.uint32) == 0)
