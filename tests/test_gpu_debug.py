"""ATTN_FWD_DEBUG: device-resident preconditions (cu_seqlens, indices,
seqlens_k) are checked before any work is launched, and a violation returns
ATTN_ERR_SHAPE.  Every test first proves that debug mode is active with a
violation that would be harmless if launched, before any case that is only
safe because the library refuses it."""

from __future__ import annotations

import numpy as np
import pytest

from synth import gen
from tests.gpu_util import dev_bf16, dev_i32, host

pytestmark = pytest.mark.gpu


def api():
    import tiled_attention_fwd_amd as t
    return t


@pytest.fixture
def debug(monkeypatch):
    monkeypatch.setenv("ATTN_FWD_DEBUG", "1")
    t = api()
    w = gen.make_varlen("dbg0", 1, [10, 6], 2, 2, 64, True)
    q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    short = dev_i32(np.array([0, 10, 15], dtype=np.int32))  # last != total (16): harmless
    with pytest.raises(t.AttnError, match="SHAPE"):
        t.attn_fwd_varlen(q, k, v, short, short, 10)
    return t


def test_consistent_inputs_run_and_match(debug, monkeypatch):
    t = debug
    w = gen.make_varlen("dbg1", 2, [70, 0, 130], 4, 2, 128, True)
    q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    cq, ck = dev_i32(w.cu_seqlens_q), dev_i32(w.cu_seqlens_k)
    o1, l1 = t.attn_fwd_varlen(q, k, v, cq, ck, w.max_seqlen, scale=float(w.scale), causal=True)
    monkeypatch.delenv("ATTN_FWD_DEBUG")
    o2, l2 = t.attn_fwd_varlen(q, k, v, cq, ck, w.max_seqlen, scale=float(w.scale), causal=True)
    assert np.array_equal(host(o1), host(o2)) and np.array_equal(host(l1), host(l2))


@pytest.mark.parametrize("cu,maxlen", [([0, 10, 8, 16], 10),    # decreasing
                                       ([1, 10, 12, 16], 10),   # does not start at 0
                                       ([0, 10, 12, 16], 9)])   # a length above max_seqlen
def test_bad_cu_seqlens(debug, cu, maxlen):
    t = debug
    w = gen.make_varlen("dbg2", 3, [10, 2, 4], 2, 2, 64, False)
    q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    bad = dev_i32(np.array(cu, dtype=np.int32))
    good = dev_i32(w.cu_seqlens_q)
    with pytest.raises(t.AttnError, match="SHAPE"):
        t.attn_fwd_varlen(q, k, v, bad, good, maxlen)
    fq = dev_i32(np.zeros(1, dtype=np.int32))
    q8 = q.view(__import__("torch").uint8)[:, :, :64].contiguous()
    with pytest.raises(t.AttnError, match="SHAPE"):
        t.attn_fwd_fp8_varlen(q8, q8, q8, bad, bad, maxlen)


def test_bad_indices_for_padded_path_and_scatter(debug):
    import torch
    t = debug
    w = gen.make_padded("dbg3", 4, 256, [128, 128], 2, 64, True, slot_lengths=[100, 50])
    q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    cu = dev_i32(w.cu_seqlens_q)
    unsorted = w.indices.copy()
    unsorted[[3, 4]] = unsorted[[4, 3]]
    with pytest.raises(t.AttnError, match="SHAPE"):
        t.attn_fwd_padded(q, k, v, dev_i32(unsorted), cu, w.max_seqlen)
    out_of_range = w.indices.copy()
    out_of_range[-1] = 256 + 7
    with pytest.raises(t.AttnError, match="SHAPE"):
        t.attn_fwd_padded(q, k, v, dev_i32(out_of_range), cu, w.max_seqlen)
    src = torch.zeros((len(w.indices), 2, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(t.AttnError, match="SHAPE"):
        t.attn_pad_scatter(src, dev_i32(unsorted), 256)


def test_padded_path_rejects_a_hole_inside_a_sequence(debug):
    """A mask with a hole inside a slot: indices are sorted and in range, but
    one sequence's rows are not consecutive, which the fused padded call needs."""
    t = debug
    w = gen.make_padded("dbg6", 7, 256, [128, 128], 2, 64, True, slot_lengths=[100, 50])
    q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    cu = dev_i32(w.cu_seqlens_q)
    holed = w.indices.copy()
    holed[60:100] += 5  # rows 60.. of slot 0 move past a 5-row hole (still < 128)
    assert np.all(np.diff(holed) > 0) and holed[99] < 128
    with pytest.raises(t.AttnError, match="SHAPE"):
        t.attn_fwd_padded(q, k, v, dev_i32(holed), cu, w.max_seqlen)
    # the same indices pass the gather, whose only precondition is order and range
    (qc,) = t.attn_unpad_gather([q], dev_i32(holed))
    assert qc.shape[0] == len(holed)
    # and the consistent padded call runs
    out, _ = t.attn_fwd_padded(q, k, v, dev_i32(w.indices), cu, w.max_seqlen)
    assert not np.isnan(host(out)).any()


def test_bad_paged_and_backward_metadata(debug):
    t = debug
    w = gen.make_paged("dbg4", 5, [1, 1], [40, 20], 4, 2, 64, 16, True)
    long_k = dev_i32(np.array([40, 41], dtype=np.int32))  # 41 > max_seqlen_k = 40
    with pytest.raises(t.AttnError, match="SHAPE"):
        t.attn_fwd_paged(dev_bf16(w.q), dev_bf16(w.k_cache), dev_bf16(w.v_cache),
                         dev_i32(w.cu_seqlens_q), long_k, dev_i32(w.block_table), 1, 40)
    vw = gen.make_varlen("dbg5", 6, [10, 6], 2, 2, 64, True)
    q, k, v = dev_bf16(vw.q), dev_bf16(vw.k), dev_bf16(vw.v)
    cq = dev_i32(vw.cu_seqlens_q)
    import torch
    out = torch.zeros(vw.q.shape, dtype=torch.float32, device="cuda")
    lse = torch.zeros((2, 16), dtype=torch.float32, device="cuda")
    bad = dev_i32(np.array([0, 12, 16], dtype=np.int32))  # lengths 12 > max_seqlen_q = 10
    with pytest.raises(t.AttnError, match="SHAPE"):
        t.attn_bwd_varlen(q, k, v, out, lse, q, bad, bad, 10, 10)
