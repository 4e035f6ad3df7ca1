"""bench.py's contract on the host: the refusal of more than one GPU, and the
work accounting behind every TFLOP/s and GB/s figure it prints (exact causal
FLOPs = 4 * D * H * visible (query, key) pairs, bottom-right causal alignment
when Lq != Lk, as in the oracle's visibility rule)."""

from __future__ import annotations

import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synth import gen  # noqa: E402


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "4"})])
def test_more_than_one_gpu_exits_with_a_message(argv, env):
    e = dict(os.environ, **env)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], env=e,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


def _visible_brute(lq, lk, causal):
    i = np.arange(lq)[:, None]
    j = np.arange(lk)[None, :]
    vis = np.ones((lq, lk), bool) if not causal else (j <= i + (lk - lq))
    return int(vis.sum())


@pytest.mark.parametrize("causal", [True, False])
def test_visible_pairs_equal_a_brute_force_count(causal):
    rng = np.random.default_rng(7)
    lq = [int(x) for x in rng.integers(0, 300, size=12)] + [1, 0, 257]
    lk = [int(x) for x in rng.integers(0, 300, size=12)] + [1, 5, 100]
    want = sum(_visible_brute(a, b, causal) for a, b in zip(lq, lk))
    assert bench.visible_pairs(lq, lk, causal) == want


def test_causal_square_pairs_closed_form():
    # a causal L x L sequence sees L (L + 1) / 2 pairs
    for L in (1, 2, 64, 2048, 8192):
        assert bench.visible_pairs([L], [L], True) == L * (L + 1) // 2


def test_attn_flops_of_configured_workloads():
    w = gen.build_workload("varlen_32x64")
    assert bench.attn_flops(w) == 4 * 128 * 16 * 32 * (64 * 65 // 2)
    # dense non-causal batch: every pair of every batch entry
    w = gen.make_dense("fl", 1, 3, 50, 70, 4, 2, 64, False)
    assert bench.attn_flops(w) == 4 * 64 * 4 * 3 * 50 * 70


def test_attn_bytes_counts_inputs_once_and_fp32_outputs():
    w = gen.make_varlen("by", 2, [10, 30], 8, 2, 64, True)
    tq = tk = 40
    want = tq * 8 * 64 * 2 + 2 * tk * 2 * 64 * 2 + tq * 8 * 64 * 4 + tq * 8 * 4
    assert bench.attn_bytes(w) == want
