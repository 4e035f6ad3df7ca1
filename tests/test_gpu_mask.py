"""GPU parity of attn_mask_to_varlen against oracle.mask_to_varlen (bit-exact
integer work), and the padded path driven end to end from a mask."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from synth import gen
from tests.gpu_util import check_o, dev_bf16, host

pytestmark = pytest.mark.gpu


def api():
    import tiled_attention_fwd_amd as t
    return t


def run(mask_np):
    import torch
    t = api()
    m = torch.from_numpy(np.ascontiguousarray(mask_np, dtype=np.uint8)).to("cuda")
    idx, cu, stats = t.attn_mask_to_varlen(m)
    st = host(stats)
    return host(idx)[:st[0]], host(cu), st


@pytest.mark.parametrize("b,l,p", [(1, 1, 1.0), (1, 4096, 0.5), (32, 128, 0.7), (3, 0, 0.5),
                                   (5, 1000, 0.0), (7, 333, 1.0), (4000, 17, 0.4),
                                   (1, 65536, 0.9), (1500, 300, 0.05)])
def test_matches_oracle(b, l, p):
    r = np.random.Generator(np.random.PCG64(b * 7 + l))
    mask = (r.random((b, l)) < p).astype(np.uint8) * r.integers(1, 256, size=(b, l), dtype=np.uint8)
    idx, cu, st = run(mask)
    i_ref, cu_ref, mx_ref = oracle.mask_to_varlen(mask)
    assert np.array_equal(idx, i_ref)
    assert np.array_equal(cu, cu_ref)
    assert st[0] == len(i_ref) and st[1] == mx_ref


def test_zero_slots():
    idx, cu, st = run(np.zeros((0, 8), dtype=np.uint8))
    assert cu.tolist() == [0] and st.tolist() == [0, 0] and idx.size == 0


def test_mask_drives_the_padded_path():
    import torch
    t = api()
    w = gen.make_padded("mk", 77, 4096, [128] * 32, 4, 128, True, random_max=128,
                        pad_value=float("nan"))
    mask = np.zeros((32, 128), dtype=np.uint8)
    for s, n in enumerate(w.lengths_q):
        mask[s, :n] = 1
    m = torch.from_numpy(mask).to("cuda")
    idx, cu, stats = t.attn_mask_to_varlen(m)
    n_valid, max_len = (int(x) for x in host(stats))  # the one host read of the path
    q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    out, lse = t.attn_fwd_padded(q, k, v, idx[:n_valid], cu, max_len, scale=float(w.scale),
                                 causal=True)
    hd = w.q.shape[2:]
    g = [oracle.unpad_gather(x, w.indices, hd) for x in (w.q, w.k, w.v)]
    o_c, _ = oracle.attention_varlen(*g, w.cu_seqlens_q, w.cu_seqlens_k, w.scale, True)
    o_ref = oracle.pad_scatter(o_c, w.indices, w.q.shape[1])
    check_o(host(out).reshape(o_ref.shape), o_ref)
