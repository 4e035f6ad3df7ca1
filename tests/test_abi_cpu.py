"""C ABI checks that need no GPU: the library loads, exports every entry point
declared in include/attn_fwd.h, and rejects bad arguments with the documented
status codes before touching the device."""

import ctypes
import os
import re

import pytest

from tiled_attention_fwd_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_fwd.h")

OK, NULL, SHAPE, UNSUP, ALIGN = 0, 1, 2, 3, 4
P = 0x100000  # a 16-byte aligned fake device address: never dereferenced by these calls


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(attn_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("attn_fwd_varlen", "attn_fwd_dense", "attn_unpad_gather", "attn_pad_scatter"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) <= set(_lib.SIGNATURES)


def test_abi_version_and_status_strings(lib):
    assert lib.attn_abi_version() == 1
    for s in range(7):
        assert lib.attn_status_str(s)
    assert b"unknown" in lib.attn_status_str(99)


def varlen(lib, **kw):
    a = dict(q=P, k=P, v=P, cq=P, ck=P, nseq=2, tq=64, tk=64, hq=4, hkv=2, d=128, maxs=32,
             scale=0.125, causal=1, out=P, lse=P)
    a.update(kw)
    return lib.attn_fwd_varlen(a["q"], a["k"], a["v"], a["cq"], a["ck"], a["nseq"], a["tq"], a["tk"],
                               a["hq"], a["hkv"], a["d"], a["maxs"], a["scale"], a["causal"],
                               a["out"], a["lse"], None)


def test_varlen_validation(lib):
    assert varlen(lib, d=48) == UNSUP
    assert varlen(lib, d=16) == UNSUP
    # every finite scale is accepted (zero and negative included); checked
    # with zero work so that nothing launches
    assert varlen(lib, scale=0.0, nseq=0) == OK
    assert varlen(lib, scale=-1.0, nseq=0) == OK
    assert varlen(lib, scale=-0.0, tq=0) == OK
    assert varlen(lib, scale=float("inf")) == UNSUP
    assert varlen(lib, scale=float("nan")) == UNSUP
    assert varlen(lib, hq=6, hkv=4) == SHAPE
    assert varlen(lib, hkv=0) == SHAPE
    assert varlen(lib, nseq=-1) == SHAPE
    assert varlen(lib, tq=-5) == SHAPE
    assert varlen(lib, maxs=0) == SHAPE
    assert varlen(lib, q=None) == NULL
    assert varlen(lib, out=None) == NULL
    assert varlen(lib, cq=None) == NULL
    assert varlen(lib, k=None) == NULL
    assert varlen(lib, q=P + 2) == ALIGN
    assert varlen(lib, out=P + 8) == ALIGN
    assert varlen(lib, lse=P + 2) == ALIGN
    # zero work succeeds without launching (no device needed)
    assert varlen(lib, nseq=0) == OK
    assert varlen(lib, tq=0) == OK
    assert varlen(lib, hq=0) == OK


def dense(lib, strides=None, **kw):
    a = dict(q=P, k=P, v=P, b=2, sq=16, sk=16, hq=4, hkv=4, d=64, scale=0.125, causal=0, out=P, lse=P)
    a.update(kw)
    return lib.attn_fwd_dense(a["q"], a["k"], a["v"], a["b"], a["sq"], a["sk"], a["hq"], a["hkv"],
                              a["d"], strides, a["scale"], a["causal"], a["out"], a["lse"], None)


def test_dense_validation(lib):
    assert dense(lib, d=96) == UNSUP
    assert dense(lib, hq=4, hkv=3) == SHAPE
    assert dense(lib, b=-1) == SHAPE
    assert dense(lib, q=None) == NULL
    assert dense(lib, v=None) == NULL
    assert dense(lib, k=P + 4) == ALIGN
    bad = (ctypes.c_int64 * 12)(*([8] * 8 + [4] + [4] * 3))
    assert dense(lib, strides=ctypes.cast(bad, ctypes.c_void_p)) == ALIGN
    neg = (ctypes.c_int64 * 12)(*([8] * 11 + [-4]))
    assert dense(lib, strides=ctypes.cast(neg, ctypes.c_void_p)) == SHAPE
    assert dense(lib, b=0) == OK
    assert dense(lib, sq=0) == OK


def test_gather_scatter_validation(lib):
    arr = (ctypes.c_void_p * 3)(P, P, P)
    pa = ctypes.cast(arr, ctypes.c_void_p)
    assert lib.attn_unpad_gather(pa, pa, 0, P, 4, 8, 256, None) == SHAPE
    assert lib.attn_unpad_gather(pa, pa, 4, P, 4, 8, 256, None) == SHAPE
    assert lib.attn_unpad_gather(pa, pa, 3, P, 4, 8, 100, None) == ALIGN
    assert lib.attn_unpad_gather(pa, pa, 3, P, -1, 8, 256, None) == SHAPE
    assert lib.attn_unpad_gather(pa, pa, 3, None, 4, 8, 256, None) == NULL
    assert lib.attn_unpad_gather(pa, pa, 3, P, 0, 8, 256, None) == OK
    mis = (ctypes.c_void_p * 3)(P, P + 8, P)
    assert lib.attn_unpad_gather(pa, ctypes.cast(mis, ctypes.c_void_p), 3, P, 4, 8, 256, None) == ALIGN
    assert lib.attn_pad_scatter(P, P, P, 5, 4, 256, None) == SHAPE
    assert lib.attn_pad_scatter(P, P, P, 4, 8, 72, None) == ALIGN
    assert lib.attn_pad_scatter(P, None, P, 4, 8, 256, None) == NULL
    assert lib.attn_pad_scatter(None, P, P, 4, 8, 256, None) == NULL
    assert lib.attn_pad_scatter(P, P, P, 0, 0, 256, None) == OK


def test_tile_override_rejects_uncompiled_policy(lib, monkeypatch):
    monkeypatch.setenv("ATTN_FWD_TILE", "2")
    assert varlen(lib, d=256) == UNSUP
    for pol in ("11", "14", "15", "16"):
        monkeypatch.setenv("ATTN_FWD_TILE", pol)
        assert varlen(lib, d=256) == UNSUP
        assert varlen(lib, d=32) == UNSUP
    monkeypatch.setenv("ATTN_FWD_TILE", "99")
    assert varlen(lib, d=128) == UNSUP


def test_workspace_plan_splits_only_low_parallelism_launches(lib, monkeypatch):
    monkeypatch.delenv("ATTN_FWD_TILE", raising=False)
    monkeypatch.delenv("ATTN_FWD_SPLIT_TILES", raising=False)
    ws = lib.attn_fwd_workspace_bytes
    # enough query blocks to occupy every CU: no split, no workspace
    assert ws(1, 2048, 16, 128, 1) == 0
    assert ws(1, 4096, 32, 128, 1) == 0
    assert ws(1, 8192, 64, 128, 1) == 0
    # few heads, long causal sequence: the key loop is split
    assert ws(1, 8192, 2, 128, 1) > 0
    assert ws(1, 16384, 1, 128, 1) > 0
    # invalid arguments report 0
    assert ws(0, 2048, 16, 128, 1) == 0
    assert ws(1, 2048, 16, 96, 1) == 0
    # forcing parts of 4 tiles sizes a workspace for any DMA-staged launch:
    # rows x blocks x parts x block x (head_dim + 1) floats
    monkeypatch.setenv("ATTN_FWD_TILE", "12")
    monkeypatch.setenv("ATTN_FWD_SPLIT_TILES", "4")
    parts = -(-(2048 // 64) // 4)
    assert ws(1, 2048, 16, 128, 1) == 16 * (2048 // 128) * parts * 128 * 129 * 4


def test_workspace_argument_checks(lib):
    P = ctypes.c_void_p(16)
    cu = ctypes.c_void_p(16)
    # negative size and misaligned workspace are rejected before any launch
    assert lib.attn_fwd_varlen_ws(P, P, P, cu, cu, 1, 8, 8, 2, 2, 64, 8, 0.125, 1, P, None,
                                  P, -1, None) == SHAPE
    assert lib.attn_fwd_varlen_ws(P, P, P, cu, cu, 1, 8, 8, 2, 2, 64, 8, 0.125, 1, P, None,
                                  ctypes.c_void_p(24), 64, None) == ALIGN
    assert lib.attn_fwd_dense_ws(P, P, P, 1, 8, 8, 2, 2, 64, None, 0.125, 1, P, None,
                                 P, -5, None) == SHAPE


def test_fused_padded_argument_checks(lib):
    P = ctypes.c_void_p(16)
    f = lib.attn_fwd_padded
    # q, k, v, indices, cu, nseq, n_valid, n_rows, hq, hkv, d, max_seqlen, scale, causal, out, lse
    assert f(P, P, P, P, P, 1, 9, 8, 2, 2, 64, 8, 0.125, 1, P, None, None) == SHAPE   # n_valid > n_rows
    assert f(P, P, P, P, P, 1, 8, 8, 2, 2, 64, 8, 0.125, 1, None, None, None) == NULL  # out
    assert f(None, P, P, P, P, 1, 8, 8, 2, 2, 64, 8, 0.125, 1, P, None, None) == NULL  # q
    assert f(P, P, P, None, P, 1, 8, 8, 2, 2, 64, 8, 0.125, 1, P, None, None) == NULL  # indices
    assert f(P, P, P, P, P, 1, 8, 8, 2, 2, 96, 8, 0.125, 1, P, None, None) == UNSUP   # head_dim
    assert f(P, P, P, P, P, 1, 8, 8, 3, 2, 64, 8, 0.125, 1, P, None, None) == SHAPE   # hq % hkv
    assert f(P, P, P, P, P, 1, 8, 8, 2, 2, 64, 0, 0.125, 1, P, None, None) == SHAPE   # max_seqlen
    assert f(P, P, P, P, P, 1, 8, 8, 2, 2, 64, 8, 0.125, 1, ctypes.c_void_p(24), None, None) == ALIGN
    assert f(P, P, P, P, P, 1, 8, 0, 2, 2, 64, 8, 0.125, 1, P, None, None) == SHAPE   # n_valid > 0 rows
    assert f(None, None, None, None, None, 0, 0, 0, 2, 2, 64, 0, 0.125, 1, None, None, None) == OK


def test_backward_argument_checks(lib):
    P = ctypes.c_void_p(16)
    f = lib.attn_bwd_varlen
    # q, k, v, out, dout, lse, cu_q, cu_k, nseq, tq, tk, hq, hkv, d, mq, mk, scale, causal,
    # dq, dk, dv, ws, ws_bytes, stream
    ok = lambda **kw: dict(dict(d=64, ws=P, wsb=1 << 20, dq=P, hq=2, hkv=2, scale=0.125, mq=8), **kw)

    def call(**kw):
        a = ok(**kw)
        return f(P, P, P, P, P, P, P, P, 1, 8, 8, a["hq"], a["hkv"], a["d"], a["mq"], 8,
                 a["scale"], 1, a["dq"], P, P, a["ws"], a["wsb"], None)
    assert call(d=48) == UNSUP and call(d=96) == UNSUP and call(d=16) == UNSUP
    assert call(scale=float("inf")) == UNSUP
    assert call(scale=float("nan")) == UNSUP
    assert call(hq=3) == SHAPE                       # hq % hkv
    assert call(wsb=8 * 2 * 4 - 4) == SHAPE          # workspace below 4 * tq * hq bytes
    assert call(wsb=-1) == SHAPE
    assert call(ws=None) == NULL
    assert call(dq=None) == NULL
    assert call(dq=ctypes.c_void_p(24)) == ALIGN
    assert call(mq=0) == SHAPE                       # queries but no max length
    assert lib.attn_bwd_workspace_bytes(8, 2) == 64
    assert lib.attn_bwd_workspace_bytes(0, 2) == 0
    g = lib.attn_bwd_dense
    assert g(P, P, P, P, P, P, 1, 8, 8, 2, 2, 96, 0.125, 1, P, P, P, P, 1 << 20, None) == UNSUP
    assert g(P, P, P, P, P, P, 1, 8, 8, 2, 2, 64, 0.125, 1, P, P, P, P, 63, None) == SHAPE
    assert g(None, None, None, None, None, None, 0, 8, 8, 2, 2, 64, 0.125, 1, None, None, None,
             None, 0, None) == OK


def test_paged_fp8_and_mask_argument_checks(lib):
    P = ctypes.c_void_p(16)
    f = lib.attn_fwd_paged

    # q, k, v, cu_q, seqlens_k, table, nseq, tq, num_pages, page_size, max_pages, hq, hkv, d,
    # max_q, max_k, scale, causal, out, lse, ws, ws_bytes, stream
    def paged(**kw):
        a = dict(dict(ps=16, d=128, mq=1, mk=32, maxp=2, hq=8, hkv=2, out=P, ws=None, wsb=0), **kw)
        return f(P, P, P, P, P, P, 2, 2, 8, a["ps"], a["maxp"], a["hq"], a["hkv"], a["d"], a["mq"],
                 a["mk"], 0.125, 1, a["out"], None, a["ws"], a["wsb"], None)
    assert paged(ps=8) == UNSUP and paged(ps=24) == UNSUP      # page size: a multiple of 16
    assert paged(d=48) == UNSUP and paged(d=96) == UNSUP
    assert paged(mk=33) == SHAPE                                # > max_pages * page_size
    assert paged(mq=0) == SHAPE
    assert paged(hq=6, hkv=4) == SHAPE
    assert paged(out=None) == NULL
    assert paged(ws=ctypes.c_void_p(24), wsb=1024) == ALIGN
    g = lib.attn_fwd_paged_fp8kv
    base = (P, P, P, P, P, P, 2, 2, 8, 16, 2, 8, 2, 128, 1, 32, 0.125)
    assert g(*base, 0.0, 1.0, 1, P, None, None, 0, None) == UNSUP   # k factor
    assert g(*base, 1.0, float("inf"), 1, P, None, None, 0, None) == UNSUP
    base48 = base[:13] + (48,) + base[14:]                       # E4M3 tiles: head_dim 32..256
    assert g(*base48, 1.0, 1.0, 1, P, None, None, 0, None) == UNSUP
    ws = lib.attn_fwd_paged_workspace_bytes
    assert ws(8, 1, 8192, 64, 8, 128) > 0                       # 64 workgroups: split in 4
    assert ws(32, 1, 8192, 64, 8, 128) == 0                     # 256 (one per CU): no split
    assert ws(32, 1, 8192, 64, 8, 96) == 0 and ws(0, 1, 8, 8, 8, 128) == 0
    h = lib.attn_fwd_fp8_varlen
    # q, k, v, cu_q, cu_k, nseq, tq, tk, hq, hkv, d, max, scale, qs, ks, vs, causal, out, lse, s
    assert h(P, P, P, P, P, 1, 8, 8, 2, 2, 96, 8, 0.125, 1.0, 1.0, 1.0, 1, P, None, None) == UNSUP
    assert h(P, P, P, P, P, 1, 8, 8, 2, 2, 64, 8, 0.125, -1.0, 1.0, 1.0, 1, P, None, None) == UNSUP
    assert h(P, P, P, P, P, 1, 8, 8, 2, 2, 64, 0, 0.125, 1.0, 1.0, 1.0, 1, P, None, None) == SHAPE
    assert h(None, P, P, P, P, 1, 8, 8, 2, 2, 64, 8, 0.125, 1.0, 1.0, 1.0, 1, P, None, None) == NULL
    d = lib.attn_fwd_fp8_dense
    assert d(P, P, P, 1, 8, 8, 2, 2, 48, 0.125, 1.0, 1.0, 1.0, 1, P, None, None) == UNSUP
    assert d(P, P, P, 0, 8, 8, 2, 2, 128, 0.125, 1.0, 1.0, 1.0, 1, None, None, None) == OK
    m = lib.attn_mask_to_varlen
    assert m(P, -1, 4, P, P, P, None) == SHAPE
    assert m(P, 1 << 16, 1 << 16, P, P, P, None) == SHAPE      # batch * seqlen >= 2^31
    assert m(P, 2, 4, P, None, P, None) == NULL
    assert m(None, 2, 4, P, P, P, None) == NULL
    assert m(P, 2, 4, P, ctypes.c_void_p(18), P, None) == ALIGN


def test_paged_noalloc_refuses_a_split_beyond_its_scratch_without_launching(lib, monkeypatch):
    """The no-allocation paged call checks its static scratch limit on the host:
    a forced one-tile-per-part split of 8000 keys over 8 KV heads needs ~126
    MiB, above the 17 MiB array, and is refused before anything touches a
    device."""
    P = ctypes.c_void_p(16)
    monkeypatch.setenv("ATTN_PAGED_CHUNK_TILES", "1")
    assert lib.attn_fwd_paged_workspace_bytes(4, 1, 8000, 32, 8, 128) > (17 << 20)
    # q, k, v, cu_q, seqlens_k, table, nseq, tq, num_pages, page_size, max_pages, hq, hkv, d,
    # max_q, max_k, scale, causal, out, lse, stream
    st = lib.attn_fwd_paged_noalloc(P, P, P, P, P, P, 4, 4, 200, 64, 125, 32, 8, 128, 1, 8000,
                                    0.125, 1, P, None, None)
    assert st == 6
    assert b"scratch" in lib.attn_status_str(6)


# The host plan for each configured workload (computed without a GPU): the
# tile policy and block order the default call launches.  A change to the
# selection shows up here first; the GPU tests then check each policy's
# results against the oracle.
PLANS = [
    # (varlen, nseq, total_q, max_seqlen, heads_q, head_dim, causal) -> policy, order, bm
    ((True, 1, 2048, 2048, 16, 128, True), (18, 1, 64)),       # bench step (b), 1 x 2048
    ((True, 32, 2048, 64, 16, 128, True), (13, 2, 128)),       # 32 x 64 packed
    ((True, 1, 8192, 8192, 16, 128, True), (19, 1, 256)),      # varlen 1 x 8192
    ((False, 1, 8192, 8192, 64, 128, True), (19, 1, 256)),     # GQA S8192, 64 query heads
    ((False, 149, 149 * 1024, 1024, 12, 64, False), (13, 3, 128)),  # ViT B149
    ((True, 1, 4096, 4096, 128, 32, True), (19, 1, 256)),      # head_dim sweep
    ((True, 1, 4096, 4096, 64, 64, True), (13, 1, 128)),
    ((True, 1, 2048, 2048, 16, 64, True), (18, 1, 64)),        # head_dim 64, few blocks: key groups
    ((True, 1, 1024, 1024, 8, 64, False), (18, 1, 64)),
    ((True, 1, 4096, 4096, 8, 64, False), (12, 1, 128)),
    ((True, 1, 4096, 4096, 32, 64, True), (12, 1, 128)),
    ((True, 1, 4096, 4096, 32, 128, True), (19, 1, 256)),
    ((True, 1, 4096, 4096, 16, 256, True), (13, 1, 128)),
    ((True, 8, 8192, 1024, 16, 256, True), (13, 2, 128)),      # head_dim 256: policy 13 throughout
    ((True, 2, 590, 300, 4, 256, False), (13, 3, 128)),
]


@pytest.mark.parametrize("shape,want", PLANS)
def test_launch_plan_of_configured_shapes(shape, want):
    import tiled_attention_fwd_amd as t
    plan = t.attn_fwd_launch_plan(*shape)
    assert (plan["policy"], plan["order"], plan["bm"]) == want, plan
