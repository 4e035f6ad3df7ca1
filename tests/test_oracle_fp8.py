"""CPU pins of the fp8 oracle (oracle/fp8.py): the E4M3 decode table against
torch's own float8_e4m3fn cast and against hand-derived values, the attention
against the (already pinned) bf16 oracle on values both formats hold exactly,
the per-tensor factors, and planted mistakes in the decode."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import oracle.fp8 as of8
from synth import gen


def torch_decode():
    b = torch.arange(256, dtype=torch.uint8)
    return b.view(torch.float8_e4m3fn).float().double().numpy()


def test_decode_table_matches_torch():
    ref = torch_decode()
    ours = of8.E4M3
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])


@pytest.mark.parametrize("byte,value", [(0x38, 1.0), (0xB8, -1.0), (0x7E, 448.0), (0x08, 2.0 ** -6),
                                        (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x80, -0.0),
                                        (0x3C, 1.5), (0x40, 2.0), (0x77, 240.0)])
def test_decode_hand_values(byte, value):
    got = of8.e4m3_to_f64(np.array([byte], dtype=np.uint8))[0]
    assert got == value and np.signbit(got) == np.signbit(value)
    assert np.isnan(of8.e4m3_to_f64(np.array([0x7F, 0xFF], dtype=np.uint8))).all()


@pytest.mark.parametrize("causal", [True, False])
def test_equals_bf16_oracle_on_shared_values(causal):
    w = gen.make_fp8_varlen("f8bf", 81, [5, 0, 37], 4, 2, 64, causal, lengths_k=[9, 3, 37])
    # every E4M3 value is exact in bf16
    to_bf16 = lambda x8: gen.bf16_bits_from_f32(of8.e4m3_to_f64(x8).astype(np.float32))
    o8, l8 = oracle.attention_fp8_varlen(w.q, w.k, w.v, w.cu_seqlens_q, w.cu_seqlens_k, w.scale,
                                         1.0, 1.0, 1.0, causal)
    ob, lb = oracle.attention_varlen(to_bf16(w.q), to_bf16(w.k), to_bf16(w.v), w.cu_seqlens_q,
                                     w.cu_seqlens_k, w.scale, causal)
    assert np.array_equal(o8, ob) and np.array_equal(l8, lb)


def test_factors_fold_into_scores_and_values():
    w = gen.make_fp8_varlen("f8sc", 82, [20, 11], 2, 2, 128, True)
    base_o, base_l = oracle.attention_fp8_varlen(w.q, w.k, w.v, w.cu_seqlens_q, w.cu_seqlens_k,
                                                 w.scale, 1.0, 1.0, 1.0, True)
    # q * 2 and k * 0.5 leave the scores unchanged; v * 4 scales the output exactly
    o, l = oracle.attention_fp8_varlen(w.q, w.k, w.v, w.cu_seqlens_q, w.cu_seqlens_k, w.scale,
                                       2.0, 0.5, 4.0, True)
    assert np.array_equal(l, base_l) and np.array_equal(o, 4.0 * base_o)


def test_dense_equals_varlen():
    r = np.random.Generator(np.random.PCG64(83))
    q = gen.normal_e4m3(r, (2, 13, 4, 64))
    k = gen.normal_e4m3(r, (2, 13, 2, 64))
    v = gen.normal_e4m3(r, (2, 13, 2, 64))
    od, ld = oracle.attention_fp8_dense(q, k, v, 0.125, 1.0, 1.0, 1.0, True)
    cu = np.array([0, 13, 26])
    ov, lv = oracle.attention_fp8_varlen(q.reshape(26, 4, 64), k.reshape(26, 2, 64),
                                         v.reshape(26, 2, 64), cu, cu, 0.125, 1.0, 1.0, 1.0, True)
    assert np.array_equal(od.reshape(26, 4, 64), ov)
    assert np.array_equal(ld.transpose(1, 0, 2).reshape(4, 26), lv)


@pytest.mark.parametrize("mutant", ["bias8", "no_subnormal", "unsigned", "nan_as_max"])
def test_decode_pins_reject_mutants(mutant):
    t = np.empty(256)
    for b in range(256):
        sign = 1.0 if mutant == "unsigned" else (-1.0 if b & 0x80 else 1.0)
        e, m = (b >> 3) & 0xF, b & 7
        bias = 8 if mutant == "bias8" else 7
        if e == 0xF and m == 7 and mutant != "nan_as_max":
            t[b] = np.nan
        elif e == 0 and mutant != "no_subnormal":
            t[b] = sign * (m / 8.0) * 2.0 ** (1 - bias)
        else:
            t[b] = sign * (1.0 + m / 8.0) * 2.0 ** (e - bias)
    ref = torch_decode()
    same = np.array_equal(np.isnan(t), np.isnan(ref)) and np.array_equal(t[~np.isnan(ref)], ref[~np.isnan(ref)])
    assert not same
