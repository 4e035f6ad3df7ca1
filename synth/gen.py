"""Seeded synthetic workloads (inputs only; no attention arithmetic here).

Every draw comes from ``numpy.random.Generator(PCG64(seed))`` in a fixed order:
sequence lengths first (when the workload has random lengths), then Q, K and V,
each as ``standard_normal(dtype=float32)`` in C order of its stated layout, then
rounded to bfloat16 with round-to-nearest-even.  Tensors are returned as
``uint16`` arrays holding the bfloat16 bit patterns, which is exactly what the
GPU library consumes and what the oracle decodes.

Layouts:
  dense   q (B, Sq, Hq, D), k/v (B, Sk, Hkv, D)
  varlen  q (Tq, Hq, D), k/v (Tk, Hkv, D) with ``cu_seqlens`` offsets
  padded  q/k/v (1, total_len, H, D) including padding rows, plus the sorted
          ``indices`` of the valid rows and the ``cu_seqlens`` of the compact
          packing that gathering those rows produces.

The workload shapes follow the attention workloads discussed on the pages
"Lesson 5: IAW model FA2 vs FA3 measured" (section 1 diagram: padded
(B=1, total_len, H, D) -> compact (total_valid, H, D) by indices; section 5
table: packed 32x64, 32x128, 1x2048, 1x8192; section 7 table: ViT 12 heads,
seq 1024, B=149) and "FlashAttention tuning: block_size and head_dim"
(head_dim measurements at seq 4096, batch 1, fixed hidden 4096).
"""

from __future__ import annotations

import dataclasses
from typing import Callable, Dict, List, Optional

import numpy as np

# Seeds per workload, fixed so every consumer sees the same bytes.
SEEDS: Dict[str, int] = {
    "varlen_32x64": 1001,
    "padded_32x128_random": 2001,
    "padded_32x128_exact": 2002,
    "padded_1x2048": 2003,
    "vit_dense_b149": 3001,
    "hdim_sweep_d32": 4032,
    "hdim_sweep_d64": 4064,
    "hdim_sweep_d128": 4128,
    "hdim_sweep_d256": 4256,
    "varlen_1x8192": 5001,
    "gqa_dense_s8192": 5002,
    "pack_64k": 5003,
}


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the upper 16 bits of the rounded float32 pattern as uint16.  NaN
    inputs map to a quiet NaN with the input's sign; infinities stay infinite.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    # 32-bit sums cannot wrap for non-NaN patterns (at most 0xFF800000 + 0x8000);
    # NaN patterns, which may wrap, are replaced below
    rounded = (bits + (np.uint32(0x7FFF) + lsb)) >> np.uint32(16)
    is_nan = (bits & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    sign = (bits >> np.uint32(16)) & np.uint32(0x8000)
    out = np.where(is_nan, sign | np.uint32(0x7FC0), rounded)
    return out.astype(np.uint16).reshape(x.shape)


def normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    """Draw N(0,1) float32 values in C order and round them to bfloat16 bits."""
    return bf16_bits_from_f32(rng.standard_normal(size=shape, dtype=np.float32))


def upstream_grad_bf16(seed: int, shape) -> np.ndarray:
    """Seeded N(0,1) bf16 bits standing in for the gradient of the attention
    output (its own stream, so the forward inputs do not change)."""
    return normal_bf16(np.random.Generator(np.random.PCG64(seed + 7_000_000)), shape)


def e4m3_bytes_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to OCP E4M3 bytes (round to nearest even) with
    torch's CPU cast; inputs must lie within +-448."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def normal_e4m3(rng: np.random.Generator, shape, sigma: float = 1.0) -> np.ndarray:
    """N(0, sigma^2) float32 draws in C order, rounded to E4M3 bytes."""
    return e4m3_bytes_from_f32(rng.standard_normal(size=shape, dtype=np.float32) * np.float32(sigma))


@dataclasses.dataclass
class Fp8Workload:
    """fp8 (E4M3) attention inputs with per-tensor dequantisation factors."""

    name: str
    causal: bool
    hq: int
    hkv: int
    d: int
    scale: np.float32
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    q_scale: np.float32
    k_scale: np.float32
    v_scale: np.float32
    cu_seqlens_q: np.ndarray
    cu_seqlens_k: np.ndarray
    lengths_q: List[int]
    lengths_k: List[int]
    max_seqlen: int
    seed: int


def make_fp8_varlen(name: str, seed: int, lengths_q, hq: int, hkv: int, d: int, causal: bool,
                    lengths_k=None, factors=(1.0, 1.0, 1.0)) -> "Fp8Workload":
    """Packed fp8 inputs; the stored bytes are N(0,1) draws divided by each
    tensor's factor, so dequantised values are N(0,1)-like."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lengths_q = [int(x) for x in lengths_q]
    lengths_k = list(lengths_q) if lengths_k is None else [int(x) for x in lengths_k]
    fq, fk, fv = (np.float32(f) for f in factors)
    q = normal_e4m3(rng, (sum(lengths_q), hq, d), 1.0 / float(fq))
    k = normal_e4m3(rng, (sum(lengths_k), hkv, d), 1.0 / float(fk))
    v = normal_e4m3(rng, (sum(lengths_k), hkv, d), 1.0 / float(fv))
    return Fp8Workload(name=name, causal=causal, hq=hq, hkv=hkv, d=d, scale=default_scale(d),
                       q=q, k=k, v=v, q_scale=fq, k_scale=fk, v_scale=fv,
                       cu_seqlens_q=cu_seqlens_from_lengths(lengths_q),
                       cu_seqlens_k=cu_seqlens_from_lengths(lengths_k), lengths_q=lengths_q,
                       lengths_k=lengths_k, max_seqlen=max(lengths_q + lengths_k + [0]), seed=seed)


def cu_seqlens_from_lengths(lengths) -> np.ndarray:
    """Packing offsets [0, L0, L0+L1, ...] as int32."""
    lens = np.asarray(lengths, dtype=np.int64)
    out = np.zeros(lens.size + 1, dtype=np.int64)
    np.cumsum(lens, out=out[1:])
    return out.astype(np.int32)


@dataclasses.dataclass
class Workload:
    """One seeded attention input set.

    ``kind`` is "dense", "varlen" or "padded".  For "padded", ``q``/``k``/``v``
    are the padded (1, total_len, H, D) tensors; ``indices`` lists the valid
    rows in increasing order; ``cu_seqlens_q``/``cu_seqlens_k`` describe the
    compact packing that gathering those rows yields.
    """

    name: str
    kind: str
    causal: bool
    hq: int
    hkv: int
    d: int
    scale: np.float32
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    seed: int
    cu_seqlens_q: Optional[np.ndarray] = None
    cu_seqlens_k: Optional[np.ndarray] = None
    max_seqlen: int = 0
    indices: Optional[np.ndarray] = None
    lengths_q: Optional[List[int]] = None
    lengths_k: Optional[List[int]] = None

    @property
    def batch(self) -> int:
        return self.q.shape[0] if self.kind == "dense" else len(self.lengths_q)


def default_scale(d: int) -> np.float32:
    return np.float32(1.0) / np.sqrt(np.float32(d))


def make_dense(name: str, seed: int, batch: int, sq: int, sk: int, hq: int, hkv: int, d: int,
               causal: bool, scale: Optional[float] = None) -> Workload:
    rng = np.random.Generator(np.random.PCG64(seed))
    q = normal_bf16(rng, (batch, sq, hq, d))
    k = normal_bf16(rng, (batch, sk, hkv, d))
    v = normal_bf16(rng, (batch, sk, hkv, d))
    return Workload(name=name, kind="dense", causal=causal, hq=hq, hkv=hkv, d=d,
                    scale=np.float32(default_scale(d) if scale is None else scale),
                    q=q, k=k, v=v, seed=seed, max_seqlen=max(sq, sk),
                    lengths_q=[sq] * batch, lengths_k=[sk] * batch)


def make_varlen(name: str, seed: int, lengths_q, hq: int, hkv: int, d: int, causal: bool,
                lengths_k=None, scale: Optional[float] = None,
                rng: Optional[np.random.Generator] = None) -> Workload:
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(seed))
    lengths_q = [int(x) for x in lengths_q]
    lengths_k = list(lengths_q) if lengths_k is None else [int(x) for x in lengths_k]
    tq, tk = sum(lengths_q), sum(lengths_k)
    q = normal_bf16(rng, (tq, hq, d))
    k = normal_bf16(rng, (tk, hkv, d))
    v = normal_bf16(rng, (tk, hkv, d))
    return Workload(name=name, kind="varlen", causal=causal, hq=hq, hkv=hkv, d=d,
                    scale=np.float32(default_scale(d) if scale is None else scale),
                    q=q, k=k, v=v, seed=seed,
                    cu_seqlens_q=cu_seqlens_from_lengths(lengths_q),
                    cu_seqlens_k=cu_seqlens_from_lengths(lengths_k),
                    max_seqlen=max(lengths_q + lengths_k + [0]),
                    lengths_q=lengths_q, lengths_k=lengths_k)


def make_padded(name: str, seed: int, total_len: int, slots, h: int, d: int, causal: bool,
                slot_lengths=None, random_max: Optional[int] = None,
                pad_value: Optional[float] = None) -> Workload:
    """Padded (1, total_len, H, D) input with valid runs at the start of each slot.

    ``slots`` lists the slot sizes (their sum must not exceed total_len; the
    rest of the rows after the last slot are padding).  Slot i holds
    ``slot_lengths[i]`` valid rows, or, when ``random_max`` is given, a length
    drawn as U{1..random_max} (drawn before the tensors).  ``pad_value``
    (e.g. NaN) overwrites every padding row after the draw.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    slots = [int(s) for s in slots]
    if sum(slots) > total_len:
        raise ValueError("slots exceed total_len")
    if random_max is not None:
        lens = [int(x) for x in rng.integers(1, random_max + 1, size=len(slots))]
    else:
        lens = [int(x) for x in slot_lengths]
    mask = np.zeros(total_len, dtype=bool)
    start = 0
    for s, L in zip(slots, lens):
        if L > s:
            raise ValueError("valid length exceeds slot")
        mask[start:start + L] = True
        start += s
    q = normal_bf16(rng, (1, total_len, h, d))
    k = normal_bf16(rng, (1, total_len, h, d))
    v = normal_bf16(rng, (1, total_len, h, d))
    if pad_value is not None:
        pad_bits = bf16_bits_from_f32(np.array([pad_value], dtype=np.float32))[0]
        for t in (q, k, v):
            t[0, ~mask] = pad_bits
    indices = np.flatnonzero(mask).astype(np.int32)
    nz = [L for L in lens if L > 0]
    return Workload(name=name, kind="padded", causal=causal, hq=h, hkv=h, d=d,
                    scale=default_scale(d), q=q, k=k, v=v, seed=seed,
                    cu_seqlens_q=cu_seqlens_from_lengths(nz),
                    cu_seqlens_k=cu_seqlens_from_lengths(nz),
                    max_seqlen=max(nz + [0]), indices=indices,
                    lengths_q=nz, lengths_k=list(nz))


@dataclasses.dataclass
class PagedWorkload:
    """New queries against a paged KV cache.

    q (Tq, Hq, D) packed by cu_seqlens_q; k_cache / v_cache (num_pages,
    page_size, Hkv, D); sequence s's key j lives in page block_table[s, j //
    page_size] at row j % page_size, for j < seqlens_k[s].  Pages are handed
    out in a random order, unused table entries are -1, and every cache row no
    sequence uses holds ``fill`` (random values, or NaN to prove it is never
    read into a result)."""

    name: str
    causal: bool
    hq: int
    hkv: int
    d: int
    scale: np.float32
    page_size: int
    q: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    block_table: np.ndarray
    seqlens_k: np.ndarray
    cu_seqlens_q: np.ndarray
    lengths_q: List[int]
    seed: int
    k_cache8: Optional[np.ndarray] = None  # E4M3 pools (fp8-cache workloads only)
    v_cache8: Optional[np.ndarray] = None

    @property
    def max_seqlen_q(self) -> int:
        return max(self.lengths_q + [0])

    @property
    def max_seqlen_k(self) -> int:
        return int(self.seqlens_k.max()) if self.seqlens_k.size else 0


def make_paged(name: str, seed: int, lengths_q, lengths_k, hq: int, hkv: int, d: int,
               page_size: int, causal: bool, spare_pages: int = 3,
               fill: Optional[float] = None) -> PagedWorkload:
    rng = np.random.Generator(np.random.PCG64(seed))
    lengths_q = [int(x) for x in lengths_q]
    lengths_k = [int(x) for x in lengths_k]
    need = [(L + page_size - 1) // page_size for L in lengths_k]
    n_pages = sum(need) + spare_pages
    max_pages = max(need + [1])
    perm = rng.permutation(n_pages)
    table = np.full((len(lengths_k), max_pages), -1, dtype=np.int32)
    at = 0
    for s, n in enumerate(need):
        table[s, :n] = perm[at:at + n]
        at += n
    q = normal_bf16(rng, (sum(lengths_q), hq, d))
    k_cache = normal_bf16(rng, (n_pages, page_size, hkv, d))
    v_cache = normal_bf16(rng, (n_pages, page_size, hkv, d))
    if fill is not None:
        used = np.zeros((n_pages, page_size), dtype=bool)
        for s, L in enumerate(lengths_k):
            j = np.arange(L)
            used[table[s, j // page_size], j % page_size] = True
        bits = bf16_bits_from_f32(np.array([fill], dtype=np.float32))[0]
        k_cache[~used] = bits
        v_cache[~used] = bits
    return PagedWorkload(name=name, causal=causal, hq=hq, hkv=hkv, d=d, scale=default_scale(d),
                         page_size=page_size, q=q, k_cache=k_cache, v_cache=v_cache,
                         block_table=table, seqlens_k=np.asarray(lengths_k, dtype=np.int32),
                         cu_seqlens_q=cu_seqlens_from_lengths(lengths_q), lengths_q=lengths_q,
                         seed=seed)


def pack_lengths_uniform(rng: np.random.Generator, total: int, max_len: int) -> List[int]:
    """Draw L ~ U{1..max_len} until the sum reaches ``total``; trim the last to hit it exactly."""
    lens: List[int] = []
    acc = 0
    while acc < total:
        L = int(rng.integers(1, max_len + 1))
        lens.append(L)
        acc += L
    lens[-1] -= acc - total
    return lens


def _pack_64k(name: str) -> Workload:
    seed = SEEDS[name]
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = pack_lengths_uniform(rng, 65536, 8192)
    return make_varlen(name, seed, lens, 16, 16, 128, True, rng=rng)


def _hdim(d: int) -> Callable[[str], Workload]:
    return lambda name: make_dense(name, SEEDS[name], 1, 4096, 4096, 4096 // d, 4096 // d, d, True)


# Full-size workloads.  Each builder takes the workload name.
WORKLOADS: Dict[str, Callable[[str], Workload]] = {
    "varlen_32x64": lambda n: make_varlen(n, SEEDS[n], [64] * 32, 16, 16, 128, True),
    "padded_32x128_random": lambda n: make_padded(n, SEEDS[n], 4096, [128] * 32, 16, 128, True,
                                                  random_max=128),
    "padded_32x128_exact": lambda n: make_padded(n, SEEDS[n], 4096, [128] * 32, 16, 128, True,
                                                 slot_lengths=[128] * 32),
    "padded_1x2048": lambda n: make_padded(n, SEEDS[n], 4096, [2048], 16, 128, True,
                                           slot_lengths=[2048]),
    "vit_dense_b149": lambda n: make_dense(n, SEEDS[n], 149, 1024, 1024, 12, 12, 64, False),
    "hdim_sweep_d32": _hdim(32),
    "hdim_sweep_d64": _hdim(64),
    "hdim_sweep_d128": _hdim(128),
    "hdim_sweep_d256": _hdim(256),
    "varlen_1x8192": lambda n: make_varlen(n, SEEDS[n], [8192], 16, 16, 128, True),
    "gqa_dense_s8192": lambda n: make_dense(n, SEEDS[n], 1, 8192, 8192, 64, 8, 128, True),
    "pack_64k": _pack_64k,
}


def build_workload(name: str) -> Workload:
    return WORKLOADS[name](name)


def _decode(b, lq, lk_range, hq, hkv, d, page):
    def build(name: str) -> PagedWorkload:
        rng = np.random.Generator(np.random.PCG64(PAGED_SEEDS[name]))
        lens = [int(x) for x in rng.integers(lk_range[0], lk_range[1] + 1, size=b)]
        return make_paged(name, PAGED_SEEDS[name] + 1, [lq] * b, lens, hq, hkv, d, page, True,
                          spare_pages=0)
    return build


# Paged KV-cache workloads (inference over a cache, page "why FA is 2x on A100
# but 1.5x on Ascend 910", section 5): decode steps of a GQA model (64 query
# heads over 8 KV heads, d=128), a long-context batch, speculative decode with
# 4 new tokens, and an MHA d=64 batch.  Key counts are drawn per sequence.
PAGED_SEEDS = {
    "decode_paged_b32_gqa8": 6001,
    "decode_paged_b8_32k": 6002,
    "specdec_paged_b32_q4": 6003,
    "decode_paged_b128_d64": 6004,
}
def _fp8kv(base: str):
    def build(name: str) -> PagedWorkload:
        w = PAGED_WORKLOADS[base](base)
        w.name = name
        w.k_cache8, w.v_cache8 = paged_cache_e4m3(w, PAGED_SEEDS[base])
        return w
    return build


PAGED_WORKLOADS: Dict[str, Callable[[str], PagedWorkload]] = {
    "decode_paged_b32_gqa8": _decode(32, 1, (4096, 8192), 64, 8, 128, 64),
    "decode_paged_b8_32k": _decode(8, 1, (32768, 32768), 64, 8, 128, 64),
    "specdec_paged_b32_q4": _decode(32, 4, (4096, 8192), 64, 8, 128, 64),
    "decode_paged_b128_d64": _decode(128, 1, (1024, 2048), 32, 32, 64, 32),
}
# the same decode batches over E4M3 caches
PAGED_WORKLOADS["decode_paged_b32_gqa8_fp8kv"] = _fp8kv("decode_paged_b32_gqa8")
PAGED_WORKLOADS["decode_paged_b8_32k_fp8kv"] = _fp8kv("decode_paged_b8_32k")


def paged_cache_e4m3(w: PagedWorkload, seed: int, factors=(1.0, 1.0)):
    """E4M3 K and V pools shaped like w's caches: N(0,1) / factor draws rounded
    to E4M3; rows no sequence owns keep the draws (or NaN bytes when w was
    made with a NaN fill)."""
    rng = np.random.Generator(np.random.PCG64(seed + 9_000_000))
    k8 = normal_e4m3(rng, w.k_cache.shape, 1.0 / float(factors[0]))
    v8 = normal_e4m3(rng, w.v_cache.shape, 1.0 / float(factors[1]))
    nan_rows = (w.k_cache == 0x7FC0) | (w.k_cache == 0xFFC0)
    k8[nan_rows] = 0x7F
    v8[nan_rows] = 0x7F
    return k8, v8


def build_paged(name: str) -> PagedWorkload:
    return PAGED_WORKLOADS[name](name)


# fp8 (E4M3) versions of the d=128 prefill workloads, plus a non-causal batch.
FP8_SEEDS = {"fp8_hdim128_s4096": 7001, "fp8_varlen_1x8192": 7002, "fp8_b4_s4096_full": 7003}
FP8_WORKLOADS: Dict[str, Callable[[str], "Fp8Workload"]] = {
    "fp8_hdim128_s4096": lambda n: make_fp8_varlen(n, FP8_SEEDS[n], [4096], 32, 32, 128, True),
    "fp8_varlen_1x8192": lambda n: make_fp8_varlen(n, FP8_SEEDS[n], [8192], 16, 16, 128, True),
    "fp8_b4_s4096_full": lambda n: make_fp8_varlen(n, FP8_SEEDS[n], [4096] * 4, 16, 16, 128, False),
}


def build_fp8(name: str) -> "Fp8Workload":
    return FP8_WORKLOADS[name](name)
