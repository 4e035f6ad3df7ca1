"""attn_fwd_paged_noalloc: the paged-cache call with the library's static
scratch instead of a caller workspace, against attn_fwd_paged with a workspace
(the same plan and kernels: bit-identical) and the fp64 oracle, on two calls in
a row, the second with a smaller input (the scratch keeps the first call's
contents).  A shape whose split needs more than the static scratch is refused
before anything is launched."""

from __future__ import annotations

import os

import numpy as np
import pytest

import oracle
from synth import gen
from tests.gpu_util import check_lse, check_o, dev_bf16, dev_i32, host

pytestmark = pytest.mark.gpu


def api():
    import tiled_attention_fwd_amd as t
    return t


def _case(w):
    import torch
    t = api()
    args = (dev_bf16(w.q), dev_bf16(w.k_cache), dev_bf16(w.v_cache), dev_i32(w.cu_seqlens_q),
            dev_i32(w.seqlens_k), dev_i32(w.block_table), w.max_seqlen_q, w.max_seqlen_k)
    nseq = len(w.lengths_q)
    need = t.attn_fwd_paged_workspace_bytes(nseq, w.max_seqlen_q, w.max_seqlen_k, w.hq, w.hkv, w.d)
    assert need > 0  # the shape splits, so the scratch is used
    tq = w.q.shape[0]
    out = torch.full((tq, w.hq, w.d), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((w.hq, tq), float("nan"), dtype=torch.float32, device="cuda")
    t.attn_fwd_paged_noalloc(*args, out=out, lse=lse, scale=float(w.scale), causal=w.causal)
    ws = t.paged_workspace(nseq, w.max_seqlen_q, w.max_seqlen_k, w.hq, w.hkv, w.d)
    o_ws, l_ws = t.attn_fwd_paged(*args, scale=float(w.scale), causal=w.causal, workspace=ws)
    torch.cuda.synchronize()
    o, l = host(out), host(lse)
    assert np.array_equal(o.view(np.uint32), host(o_ws).view(np.uint32))
    assert np.array_equal(l.view(np.uint32), host(l_ws).view(np.uint32))
    o_ref, l_ref = oracle.attention_paged(w.q, w.k_cache, w.v_cache, w.cu_seqlens_q, w.seqlens_k,
                                          w.block_table, w.scale, w.causal)
    return check_o(o, o_ref), check_lse(l, l_ref)


def test_noalloc_two_calls_second_smaller():
    assert "ATTN_PAGED_CHUNK_TILES" not in os.environ
    big = gen.make_paged("na1", 8101, [1] * 16, list(range(2000, 2000 + 16 * 61, 61)), 64, 8, 128,
                         64, True, fill=float("nan"))
    small = gen.make_paged("na2", 8102, [2, 1, 3, 1], [900, 77, 1500, 33], 16, 4, 128, 32, True,
                           fill=float("nan"))
    print("first", _case(big))
    print("second", _case(small))


def test_noalloc_refuses_a_split_beyond_its_scratch():
    import torch
    t = api()
    w = gen.make_paged("na3", 8103, [1] * 4, [8000, 100, 3000, 50], 32, 8, 128, 64, True)
    out = torch.zeros((w.q.shape[0], w.hq, w.d), dtype=torch.float32, device="cuda")
    args = (dev_bf16(w.q), dev_bf16(w.k_cache), dev_bf16(w.v_cache), dev_i32(w.cu_seqlens_q),
            dev_i32(w.seqlens_k), dev_i32(w.block_table), w.max_seqlen_q, w.max_seqlen_k)
    os.environ["ATTN_PAGED_CHUNK_TILES"] = "1"  # one part per 32-key tile: far above the scratch
    try:
        nseq = len(w.lengths_q)
        assert t.attn_fwd_paged_workspace_bytes(nseq, 1, w.max_seqlen_k, w.hq, w.hkv,
                                                w.d) > (17 << 20)
        with pytest.raises(t.AttnError, match="SCRATCH"):
            t.attn_fwd_paged_noalloc(*args, out=out, scale=float(w.scale), causal=True)
    finally:
        os.environ.pop("ATTN_PAGED_CHUNK_TILES", None)
    torch.cuda.synchronize()
    assert float(out.abs().max()) == 0.0  # nothing was launched
    # the default plan of the same shape runs
    t.attn_fwd_paged_noalloc(*args, out=out, scale=float(w.scale), causal=True)
    o_ref, _ = oracle.attention_paged(w.q, w.k_cache, w.v_cache, w.cu_seqlens_q, w.seqlens_k,
                                      w.block_table, w.scale, True)
    check_o(host(out), o_ref)
