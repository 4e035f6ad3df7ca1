"""CPU pins of the paged-KV oracle (oracle/paged.py).

None of these re-types the oracle: a pure-Python loop that follows the page
table key by key, a layout that reduces paged attention to the dense and
varlen oracles (already pinned), the Q = 0 closed form on a hand-worked page
table (tests/golden/paged_q0.json), invariance under relabelling the physical
pages, isolation from cache rows no sequence owns, and planted mistakes that
these pins must reject.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest

import oracle
import oracle.paged as opg
from oracle.attention import bf16_bits_to_f64
from synth import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "paged_q0.json")


def brute(w):
    """Per (sequence, head, query): walk the page table one key at a time."""
    q = bf16_bits_to_f64(w.q)
    kc = bf16_bits_to_f64(w.k_cache)
    vc = bf16_bits_to_f64(w.v_cache)
    group = w.hq // w.hkv
    out = np.zeros(q.shape)
    lse = np.full((w.hq, q.shape[0]), -np.inf)
    sc = float(np.float32(w.scale))
    for s in range(len(w.lengths_q)):
        q0, lq, lk = int(w.cu_seqlens_q[s]), w.lengths_q[s], int(w.seqlens_k[s])
        for h in range(w.hq):
            g = h // group
            for i in range(lq):
                keys = []
                for j in range(lk):
                    if w.causal and j > i + lk - lq:
                        continue
                    page = int(w.block_table[s][j // w.page_size])
                    row = j % w.page_size
                    keys.append((kc[page, row, g], vc[page, row, g]))
                if not keys:
                    continue
                scores = [sc * math.fsum(float(a) * float(b) for a, b in zip(q[q0 + i, h], kk))
                          for kk, _ in keys]
                m = max(scores)
                e = [math.exp(x - m) for x in scores]
                l = math.fsum(e)
                for dd in range(q.shape[2]):
                    out[q0 + i, h, dd] = math.fsum(ei * float(vv[dd]) for ei, (_, vv) in zip(e, keys)) / l
                lse[h, q0 + i] = m + math.log(l)
    return out, lse


def run(w, fn=oracle.attention_paged):
    return fn(w.q, w.k_cache, w.v_cache, w.cu_seqlens_q, w.seqlens_k, w.block_table, w.scale,
              w.causal)


CASES = [
    ("decode", [1, 1, 1], [13, 1, 40], 4, 2, 8, 4, True),
    ("spec", [3, 2], [9, 2], 2, 1, 16, 4, True),
    ("lq>lk", [5], [3], 2, 2, 8, 2, True),
    ("noncausal", [2, 4], [7, 16], 3, 3, 8, 8, False),
    ("empty", [2, 0, 1], [0, 5, 6], 2, 1, 8, 4, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_matches_page_table_walk(case):
    name, lq, lk, hq, hkv, d, ps, causal = case
    w = gen.make_paged(name, 31, lq, lk, hq, hkv, d, ps, causal)
    o, lse = run(w)
    ob, lb = brute(w)
    assert np.allclose(o, ob, atol=1e-12, rtol=1e-12)
    fin = np.isfinite(lb)
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.allclose(lse[fin], lb[fin], atol=1e-12)


def test_one_page_per_sequence_is_the_dense_layout():
    # cache (B, L, Hkv, D) with page_size = L and block_table[b] = [b]
    b, lq, lk, hq, hkv, d = 3, 6, 10, 4, 2, 16
    r = np.random.Generator(np.random.PCG64(5))
    q = gen.normal_bf16(r, (b, lq, hq, d))
    k = gen.normal_bf16(r, (b, lk, hkv, d))
    v = gen.normal_bf16(r, (b, lk, hkv, d))
    for causal in (True, False):
        od, ld = oracle.attention_dense(q, k, v, 0.25, causal)
        op, lp = oracle.attention_paged(q.reshape(b * lq, hq, d), k, v,
                                        gen.cu_seqlens_from_lengths([lq] * b),
                                        np.full(b, lk), np.arange(b).reshape(b, 1), 0.25, causal)
        assert np.array_equal(op, od.reshape(b * lq, hq, d))
        assert np.array_equal(lp, ld.transpose(1, 0, 2).reshape(hq, b * lq))


def test_packed_cache_equals_varlen():
    # page_size 1 and the identity table: the cache is the packed (Tk, Hkv, D) tensor
    w = gen.make_varlen("pv", 41, [4, 1, 7], 4, 2, 8, True, lengths_k=[9, 6, 7])
    ck = w.cu_seqlens_k
    table = np.full((3, 9), -1)
    for s in range(3):
        table[s, :ck[s + 1] - ck[s]] = np.arange(ck[s], ck[s + 1])
    op, lp = oracle.attention_paged(w.q, w.k[:, None], w.v[:, None], w.cu_seqlens_q,
                                    np.diff(ck), table, w.scale, True)
    ov, lv = oracle.attention_varlen(w.q, w.k, w.v, w.cu_seqlens_q, ck, w.scale, True)
    assert np.array_equal(op, ov) and np.array_equal(lp, lv)


def test_q0_golden():
    g = json.load(open(GOLDEN))
    kc = np.array(g["k_cache"], dtype=np.float32)
    vc = np.array(g["v_cache"], dtype=np.float32)
    o, lse = oracle.attention_paged(
        gen.bf16_bits_from_f32(np.zeros((1, 1, kc.shape[-1]), np.float32)),
        gen.bf16_bits_from_f32(kc), gen.bf16_bits_from_f32(vc), [0, 1], [g["seqlen"]],
        np.array([g["block_table"]]), 1.0, True)
    assert np.allclose(o[0, 0], g["expected_out"], atol=1e-12)
    assert abs(lse[0, 0] - math.log(g["seqlen"])) < 1e-12


def test_relabelling_pages_changes_nothing():
    w = gen.make_paged("perm", 51, [2, 1], [19, 30], 4, 2, 8, 4, True)
    o, lse = run(w)
    perm = np.random.Generator(np.random.PCG64(3)).permutation(w.k_cache.shape[0])
    inv = np.argsort(perm)            # new page p holds old page perm[p]
    w2 = gen.make_paged("perm", 51, [2, 1], [19, 30], 4, 2, 8, 4, True)
    w2.k_cache = w.k_cache[perm]
    w2.v_cache = w.v_cache[perm]
    w2.block_table = np.where(w.block_table >= 0, inv[np.maximum(w.block_table, 0)], -1)
    o2, lse2 = run(w2)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_rows_no_sequence_owns_are_never_read():
    a = gen.make_paged("iso", 61, [1, 2], [11, 6], 2, 2, 8, 4, True)
    b = gen.make_paged("iso", 61, [1, 2], [11, 6], 2, 2, 8, 4, True, fill=float("nan"))
    oa, la = run(a)
    ob, lb = run(b)
    assert np.isfinite(ob).all()
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)


# ------------------------------------------------------------------ planted mistakes
def _mutant(kind):
    def gather(cache, row, seqlen):
        ps = cache.shape[1]
        j = np.arange(seqlen)
        table = np.asarray(row, dtype=np.int64)
        if kind == "page_by_position":        # ignore the table
            return cache[j // ps, j % ps]
        if kind == "row_from_quotient":       # swapped div / mod
            return cache[table[j % ps % len(table)], (j // ps) % ps]
        if kind == "one_short":               # drops the last key
            j = j[:-1]
        return cache[table[j // ps], j % ps]

    def paged(q_bits, kc, vc, cu_q, seqlens_k, table, scale, causal):
        saved = opg.gather_pages
        opg.gather_pages = gather
        try:
            if kind == "top_left_causal":
                return _top_left(q_bits, kc, vc, cu_q, seqlens_k, table, scale)
            return opg.attention_paged(q_bits, kc, vc, cu_q, seqlens_k, table, scale, causal)
        finally:
            opg.gather_pages = saved
    return paged


def _top_left(q_bits, kc, vc, cu_q, seqlens_k, table, scale):
    q = bf16_bits_to_f64(q_bits)
    o = np.zeros(q.shape)
    lse = np.full((q.shape[1], q.shape[0]), -np.inf)
    group = q.shape[1] // kc.shape[2]
    for s in range(len(cu_q) - 1):
        q0, q1 = int(cu_q[s]), int(cu_q[s + 1])
        k = bf16_bits_to_f64(opg.gather_pages(kc, table[s], int(seqlens_k[s])))
        v = bf16_bits_to_f64(opg.gather_pages(vc, table[s], int(seqlens_k[s])))
        for h in range(q.shape[1]):
            g = h // group
            lq = q1 - q0
            # mistake: aligns the diagonal to the first key instead of the last
            o[q0:q1, h], lse[h, q0:q1] = oracle.attention_one(q[q0:q1, h], k[:lq, g], v[:lq, g],
                                                              np.float32(scale), True)
    return o, lse


@pytest.mark.parametrize("kind", ["page_by_position", "row_from_quotient", "one_short",
                                  "top_left_causal"])
def test_pins_reject_planted_mistakes(kind):
    w = gen.make_paged("mut", 71, [2, 1], [10, 7], 2, 1, 8, 4, True)
    o, lse = _mutant(kind)(w.q, w.k_cache, w.v_cache, w.cu_seqlens_q, w.seqlens_k,
                           w.block_table, w.scale, True)
    ob, lb = brute(w)
    assert not np.allclose(o, ob, atol=1e-9)


def test_fp8kv_equals_bf16_oracle_on_shared_values():
    # every E4M3 value is exact in bf16, so the fp8 cache oracle must equal the
    # (pinned) bf16 paged oracle on the same values, with factors applied exactly
    import oracle.fp8 as of8
    w = gen.make_paged("f8kv", 91, [1, 3, 2], [40, 9, 33], 8, 2, 64, 16, True)
    k8, v8 = gen.paged_cache_e4m3(w, 91)
    to_bf16 = lambda x8, f: gen.bf16_bits_from_f32((of8.e4m3_to_f64(x8) * f).astype(np.float32))
    for kf, vf in ((1.0, 1.0), (0.5, 4.0)):
        o8, l8 = oracle.attention_paged_fp8kv(w.q, k8, v8, w.cu_seqlens_q, w.seqlens_k,
                                              w.block_table, w.scale, kf, vf, True)
        ob, lb = oracle.attention_paged(w.q, to_bf16(k8, kf), to_bf16(v8, vf), w.cu_seqlens_q,
                                        w.seqlens_k, w.block_table, w.scale, True)
        assert np.array_equal(o8, ob) and np.array_equal(l8, lb)


def test_fp8kv_unowned_nan_rows_never_read():
    w = gen.make_paged("f8nan", 92, [1, 2], [21, 6], 4, 2, 64, 16, True, fill=float("nan"))
    k8, v8 = gen.paged_cache_e4m3(w, 92)
    assert (k8 == 0x7F).any()
    o, lse = oracle.attention_paged_fp8kv(w.q, k8, v8, w.cu_seqlens_q, w.seqlens_k,
                                          w.block_table, w.scale, 1.0, 1.0, True)
    assert np.isfinite(o).all()
