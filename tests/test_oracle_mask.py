"""CPU pins of oracle.mask_to_varlen: a hand-worked golden example, a
pure-Python row loop on random masks, consistency with the padded workloads'
own index lists, and planted mistakes that must fail."""

from __future__ import annotations

import json
import os

import numpy as np
import pytest

import oracle
from synth import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mask_to_varlen_example.json")


def loop(mask):
    idx, cu, mx = [], [0], 0
    for b, row in enumerate(mask):
        n = 0
        for i, v in enumerate(row):
            if v != 0:
                idx.append(b * len(row) + i)
                n += 1
        cu.append(cu[-1] + n)
        mx = max(mx, n)
    return idx, cu, mx


def test_golden():
    g = json.load(open(GOLDEN))
    idx, cu, mx = oracle.mask_to_varlen(np.array(g["mask"], dtype=np.uint8))
    assert idx.tolist() == g["indices"] and cu.tolist() == g["cu_seqlens"] and mx == g["max_seqlen"]


@pytest.mark.parametrize("b,l,p", [(1, 1, 0.5), (3, 17, 0.0), (5, 64, 1.0), (33, 129, 0.3), (7, 1000, 0.9)])
def test_against_row_loop(b, l, p):
    r = np.random.Generator(np.random.PCG64(b * 1000 + l))
    mask = (r.random((b, l)) < p).astype(np.uint8) * r.integers(1, 256, size=(b, l), dtype=np.uint8)
    idx, cu, mx = oracle.mask_to_varlen(mask)
    i2, c2, m2 = loop(mask)
    assert idx.tolist() == i2 and cu.tolist() == c2 and mx == m2
    assert idx.dtype == np.int32 and cu.dtype == np.int32


def test_matches_padded_workload_layout():
    # make_padded lays out slots of 128 rows with valid runs at their starts and
    # lists the valid rows itself; the mask of those runs must give the same rows
    w = gen.make_padded("m", 5, 4096, [128] * 32, 2, 64, True, random_max=128)
    mask = np.zeros((32, 128), dtype=np.uint8)
    for s, n in enumerate(w.lengths_q):
        mask[s, :n] = 1
    idx, cu, mx = oracle.mask_to_varlen(mask)
    assert np.array_equal(idx, w.indices)
    assert np.array_equal(cu, w.cu_seqlens_q) and mx == w.max_seqlen


@pytest.mark.parametrize("mutant", ["column_major", "counts_off_by_one", "max_of_cu"])
def test_pins_reject_mutants(mutant):
    g = json.load(open(GOLDEN))
    mask = np.array(g["mask"], dtype=np.uint8)
    if mutant == "column_major":
        idx = np.flatnonzero(mask.T.reshape(-1)).astype(np.int32)
        ok = idx.tolist() == g["indices"]
    elif mutant == "counts_off_by_one":
        cu = np.concatenate([[0], np.cumsum((mask != 0).sum(1) - 1)])
        ok = cu.tolist() == g["cu_seqlens"]
    else:
        cu = np.concatenate([[0], np.cumsum((mask != 0).sum(1))])
        ok = int(cu.max()) == g["max_seqlen"]
    assert not ok
