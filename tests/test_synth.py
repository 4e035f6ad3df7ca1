"""Seeded input generators: bf16 rounding against hand-computed bit patterns,
determinism, and packing descriptors."""

import numpy as np

from synth import gen


def test_bf16_round_to_nearest_even_bit_patterns():
    f32 = np.array([0x3F800000,   # 1.0 -> 0x3F80
                    0x3F808000,   # halfway, lower even -> 0x3F80
                    0x3F818000,   # halfway, upper even -> 0x3F82
                    0x3F808001,   # just above halfway -> 0x3F81
                    0x3F807FFF,   # just below halfway -> 0x3F80
                    0x7F800000,   # +inf
                    0xFF800000,   # -inf
                    0x7FC00001,   # NaN stays NaN
                    0x80000000,   # -0.0
                    0x00000001,   # smallest subnormal rounds to +0
                    0x7F7FFFFF,   # max float rounds up to +inf
                    ], dtype=np.uint32).view(np.float32)
    want = np.array([0x3F80, 0x3F80, 0x3F82, 0x3F81, 0x3F80, 0x7F80, 0xFF80, 0x7FC0, 0x8000,
                     0x0000, 0x7F80], dtype=np.uint16)
    assert np.array_equal(gen.bf16_bits_from_f32(f32), want)


def test_generators_are_deterministic():
    a = gen.make_varlen("x", 7, [3, 5], 2, 1, 32, True)
    b = gen.make_varlen("x", 7, [3, 5], 2, 1, 32, True)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.k, b.k) and np.array_equal(a.v, b.v)
    c = gen.make_varlen("x", 8, [3, 5], 2, 1, 32, True)
    assert not np.array_equal(a.q, c.q)


def test_packing_descriptors():
    assert gen.cu_seqlens_from_lengths([64] * 32).tolist() == list(range(0, 2049, 64))
    w = gen.make_padded("p", 3, 64, [16, 16, 16, 16], 2, 32, True, random_max=16)
    assert np.all(np.diff(w.indices) > 0)
    assert w.cu_seqlens_q[-1] == len(w.indices)
    assert sum(w.lengths_q) == len(w.indices)
    r = np.random.Generator(np.random.PCG64(5))
    lens = gen.pack_lengths_uniform(r, 65536, 8192)
    assert sum(lens) == 65536 and min(lens) >= 1 and max(lens) <= 8192


def test_full_size_shapes_small_ones_only():
    w = gen.build_workload("varlen_32x64")
    assert w.q.shape == (2048, 16, 128) and w.q.dtype == np.uint16
    assert w.cu_seqlens_q.tolist() == list(range(0, 2049, 64))
    p = gen.build_workload("padded_1x2048")
    assert p.q.shape == (1, 4096, 16, 128) and p.indices.tolist() == list(range(2048))
