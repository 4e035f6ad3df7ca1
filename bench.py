#!/usr/bin/env python3
"""Benchmark of the FlashAttention forward hot path on one MI355X.

One step = the packed LLM path with padding (page "Lesson 5: IAW model FA2 vs
FA3 measured", section 1) over both input variants of that workload:
  (a) B=1, total_len 4096, 32 slots of 128 positions, valid lengths U{1..128}
  (b) B=1, total_len 4096, one sequence of 2048 valid rows, 2048 padding rows
each as unpad gather of q, k, v (one launch) -> causal varlen attention
(H=16, D=128, bf16) -> pad scatter of the fp32 output (one launch).

Printed: ONE JSON line.  `value` is attention TFLOP/s of the whole step (exact
causal FLOPs = 4 * D * H * visible (query, key) pairs, divided by the wall time
of K back-to-back steps with inputs resident in HBM).  `roofline` reports the
kernel that takes the most time per step; its average launch duration comes
from HIP events on the launch stream around batches of its launches.
`cpu_baseline` times the fp64 oracle on the host for the same step.
`configs` adds one row per listed workload (cold-cache per-call timing).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["tiled_attention_fwd_amd/csrc/attn_device.h",
                  "tiled_attention_fwd_amd/csrc/attn_kernel.hip",
                  "tiled_attention_fwd_amd/csrc/attn_kernel_d256.hip",
                  "tiled_attention_fwd_amd/csrc/rows_kernel.hip"]


# ------------------------------------------------------------------------- work accounting
def visible_pairs(lengths_q, lengths_k, causal):
    tot = 0
    for lq, lk in zip(lengths_q, lengths_k):
        if not causal:
            tot += lq * lk
        else:
            off = lk - lq
            # rows i see min(lk, max(0, i + off + 1)) keys
            for i in range(lq):
                tot += min(lk, max(0, i + off + 1))
    return tot


def attn_flops(w):
    return 4 * w.d * w.hq * visible_pairs(w.lengths_q, w.lengths_k, w.causal)


def attn_bytes(w):
    tq, tk = sum(w.lengths_q), sum(w.lengths_k)
    return (tq * w.hq * w.d * 2 + 2 * tk * w.hkv * w.d * 2 + tq * w.hq * w.d * 4 + tq * w.hq * 4)


def source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(kernel_tag):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(PROFILES, f"traffic_{kernel_tag}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_hash") != source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ------------------------------------------------------------------------- GPU plumbing
class PaddedPath:
    """Device buffers for one padded-path input, allocated once."""

    def __init__(self, w, torch, t):
        import numpy as np
        self.w, self.t = w, t
        dev = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to("cuda").view(torch.bfloat16)
        self.q, self.k, self.v = dev(w.q), dev(w.k), dev(w.v)
        self.idx = torch.from_numpy(w.indices).to("cuda")
        self.cu = torch.from_numpy(w.cu_seqlens_q).to("cuda")
        n = len(w.indices)
        h, d = w.hq, w.d
        self.qc = torch.empty((n, h, d), dtype=torch.bfloat16, device="cuda")
        self.kc = torch.empty_like(self.qc)
        self.vc = torch.empty_like(self.qc)
        self.o = torch.empty((n, h, d), dtype=torch.float32, device="cuda")
        self.lse = torch.empty((h, n), dtype=torch.float32, device="cuda")
        self.total_len = w.q.shape[1]
        self.out = torch.empty((1, self.total_len, h, d), dtype=torch.float32, device="cuda")
        self.n_valid = n
        # workspace for split key ranges (None when the shape is not split)
        self.ws = t.workspace(len(w.lengths_q), w.max_seqlen, h, d, True)
        self.out_f = torch.empty_like(self.out)
        self.lse_f = torch.empty_like(self.lse)

    def gather(self):
        self.t.attn_unpad_gather([self.q, self.k, self.v], self.idx, outs=[self.qc, self.kc, self.vc])

    def attention(self):
        self.t.attn_fwd_varlen(self.qc, self.kc, self.vc, self.cu, self.cu, self.w.max_seqlen,
                               scale=float(self.w.scale), causal=True, out=self.o, lse=self.lse,
                               workspace=self.ws)

    def scatter(self):
        self.t.attn_pad_scatter(self.o, self.idx, self.total_len, out=self.out)

    def fused(self):
        """The same padded input and output through attn_fwd_padded (no compact copies)."""
        self.t.attn_fwd_padded(self.q, self.k, self.v, self.idx, self.cu, self.w.max_seqlen,
                               scale=float(self.w.scale), causal=True, out=self.out_f,
                               lse=self.lse_f)

    def bytes_gather(self):
        return 3 * 2 * self.n_valid * self.w.hq * self.w.d * 2

    def bytes_scatter(self):
        row = self.w.hq * self.w.d * 4
        return self.n_valid * row + self.total_len * row


def spin(torch):
    """Queues ~0.5 ms of GPU spinning so that the host can enqueue the next
    launches before the GPU reaches them (event pairs then bracket kernels only)."""
    try:
        torch.cuda._sleep(1_200_000)
    except Exception:  # pragma: no cover
        x = torch.empty((4096, 4096), device="cuda", dtype=torch.bfloat16)
        x @ x


class CacheFlush:
    """Cold-cache set-up: one pass over a 1 GiB buffer (more than MALL + L2)
    evicts every input of the next call.  The pass reads, so the caches are
    left holding clean lines only.  A writing pass would leave up to MALL + L2
    of dirty lines, and their write-back to HBM would run inside the next
    timed call and compete with it for bandwidth; `write()` is that pass,
    kept for comparison."""

    def __init__(self, torch):
        self.buf = torch.zeros(1 << 28, dtype=torch.float32, device="cuda")

    def __call__(self):
        self.buf.sum()

    def write(self):
        self.buf.zero_()


def time_calls(torch, fn, iters, warmup, flush=None):
    """Per-call device time (us) with events.  Before each call either `flush`
    (a pass over 1 GiB that evicts L2 and MALL: cold) or a spin kernel (warm)
    runs."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    times = []
    s = torch.cuda.current_stream()
    for _ in range(iters):
        if flush is not None:
            flush()
        else:
            spin(torch)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(s)
        fn()
        b.record(s)
        b.synchronize()
        times.append(a.elapsed_time(b) * 1000.0)
    return times


def run_configs(torch, t, names, flush, oracle_budget_s=0.0):
    """Per-workload cold and warm call times; with oracle_budget_s > 0 each row
    also gets the fp64 oracle's time for the same workload on the host."""
    import numpy as np
    from synth import gen
    rows = []
    for name in names:
        w = gen.build_workload(name)
        dev = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to("cuda").view(torch.bfloat16)
        q, k, v = dev(w.q), dev(w.k), dev(w.v)
        if w.kind == "padded":
            # the whole padded path as one span: gather q,k,v -> attention -> scatter
            pp = PaddedPath(w, torch, t)
            o, lse = pp.o, pp.lse

            def fn(pp=pp):
                pp.gather()
                pp.attention()
                pp.scatter()
        elif w.kind == "dense":
            o = torch.empty(w.q.shape, dtype=torch.float32, device="cuda")
            lse = torch.empty((w.q.shape[0], w.hq, w.q.shape[1]), dtype=torch.float32, device="cuda")
            ws = t.workspace(w.q.shape[0], w.q.shape[1], w.hq, w.d, w.causal)
            fn = lambda: t.attn_fwd_dense(q, k, v, scale=float(w.scale), causal=w.causal, out=o,
                                          lse=lse, workspace=ws)
        else:
            cq = torch.from_numpy(w.cu_seqlens_q).to("cuda")
            ck = torch.from_numpy(w.cu_seqlens_k).to("cuda")
            o = torch.empty(w.q.shape, dtype=torch.float32, device="cuda")
            lse = torch.empty((w.hq, w.q.shape[0]), dtype=torch.float32, device="cuda")
            ws = t.workspace(len(w.lengths_q), w.max_seqlen, w.hq, w.d, w.causal)
            fn = lambda: t.attn_fwd_varlen(q, k, v, cq, ck, w.max_seqlen, scale=float(w.scale),
                                           causal=w.causal, out=o, lse=lse, workspace=ws)
        fl, by = attn_flops(w), attn_bytes(w)
        if w.kind == "padded":
            by = by + pp.bytes_gather() + pp.bytes_scatter()
        probe = time_calls(torch, fn, 3, 2)
        iters = int(min(50, max(5, 0.25e6 / max(1.0, statistics.median(probe)))))
        cold = time_calls(torch, fn, iters, 1, flush=flush)
        warm = time_calls(torch, fn, iters, 1)
        med = statistics.median(cold)
        tf = fl / (med * 1e-6) / 1e12
        gbs = by / (med * 1e-6) / 1e9
        t_mfma = fl / (PEAK_BF16_TFLOPS * 1e12) * 1e6
        t_hbm = by / (PEAK_HBM_GBS * 1e9) * 1e6
        rows.append({
            "workload": name, "us_median_cold": round(med, 2),
            "us_p10": round(sorted(cold)[len(cold) // 10], 2),
            "us_p90": round(sorted(cold)[(len(cold) * 9) // 10], 2),
            "us_median_warm": round(statistics.median(warm), 2),
            "gflop": round(fl / 1e9, 3), "tflops": round(tf, 1),
            "pct_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 1),
            "gbs": round(gbs, 1), "pct_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 1),
            "bound": "mfma" if t_mfma >= t_hbm else "hbm",
            "pct_of_bound": round(100 * max(t_mfma, t_hbm) / med, 1),
        })
        if oracle_budget_s > 0:
            orc = oracle_config_time(w, oracle_budget_s)
            orc["gpu_speedup"] = round(orc["s"] / (med * 1e-6), 1)
            rows[-1]["oracle"] = orc
        del q, k, v, o, lse
        torch.cuda.empty_cache()
    return rows


def run_backward(torch, t, names, flush):
    """Backward (attn_bwd_*) per workload: the forward runs once for out/lse,
    then the three backward launches are timed as one call.  FLOPs follow the
    usual convention of 2.5x the forward (five products of the visible
    pairs); the kernels execute seven (S and dP are recomputed in both the dQ
    and the dK/dV pass, which keeps the passes free of atomics)."""
    import numpy as np
    from synth import gen
    rows = []
    for name in names:
        w = gen.build_workload(name)
        if w.d not in (32, 64, 128, 256) or w.kind == "padded":
            continue
        dev = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to("cuda").view(torch.bfloat16)
        q, k, v = dev(w.q), dev(w.k), dev(w.v)
        do = dev(gen.upstream_grad_bf16(w.seed, w.q.shape))
        dq = torch.empty(w.q.shape, dtype=torch.float32, device="cuda")
        dk = torch.empty(w.k.shape, dtype=torch.float32, device="cuda")
        dv = torch.empty(w.v.shape, dtype=torch.float32, device="cuda")
        if w.kind == "dense":
            o, lse = t.attn_fwd_dense(q, k, v, scale=float(w.scale), causal=w.causal)
            ws = torch.empty(t.attn_bwd_workspace_bytes(w.q.shape[0] * w.q.shape[1], w.hq),
                             dtype=torch.uint8, device="cuda")
            fn = lambda: t.attn_bwd_dense(q, k, v, o, lse, do, scale=float(w.scale),
                                          causal=w.causal, dq=dq, dk=dk, dv=dv, workspace=ws)
        else:
            cq = torch.from_numpy(w.cu_seqlens_q).to("cuda")
            ck = torch.from_numpy(w.cu_seqlens_k).to("cuda")
            o, lse = t.attn_fwd_varlen(q, k, v, cq, ck, w.max_seqlen, scale=float(w.scale),
                                       causal=w.causal)
            ws = torch.empty(t.attn_bwd_workspace_bytes(w.q.shape[0], w.hq), dtype=torch.uint8,
                             device="cuda")
            fn = lambda: t.attn_bwd_varlen(q, k, v, o, lse, do, cq, ck, w.max_seqlen, w.max_seqlen,
                                           scale=float(w.scale), causal=w.causal, dq=dq, dk=dk,
                                           dv=dv, workspace=ws)
        fl = 2.5 * attn_flops(w)
        probe = time_calls(torch, fn, 3, 2)
        iters = int(min(30, max(5, 0.25e6 / max(1.0, statistics.median(probe)))))
        cold = time_calls(torch, fn, iters, 1, flush=flush)
        med = statistics.median(cold)
        tf = fl / (med * 1e-6) / 1e12
        rows.append({"workload": name, "us_median_cold": round(med, 1), "gflop": round(fl / 1e9, 2),
                     "tflops": round(tf, 1), "pct_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 1),
                     # products executed: S and dP in both the dQ and dK/dV passes (7 of
                     # the 5 the gradient needs); at head_dim 256 S a third time (dV and
                     # dK run as separate passes)
                     "executed_tflops": round(tf * (8 if w.d == 256 else 7) / 5, 1)})
        del q, k, v, o, lse, do, dq, dk, dv, ws
        torch.cuda.empty_cache()
    return rows


def run_paged(torch, t, names, flush):
    """attn_fwd_paged per paged-cache workload (with its split workspace).
    The bound is HBM: algorithmic bytes are K and V of every sequence read
    once per KV head, q read once, out (fp32) and lse written once."""
    import numpy as np
    from synth import gen
    rows = []
    for name in names:
        w = gen.build_paged(name)
        dev = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to("cuda").view(torch.bfloat16)
        i32 = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to("cuda")
        fp8kv = w.k_cache8 is not None
        u8 = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda")
        q = dev(w.q)
        kc, vc = (u8(w.k_cache8), u8(w.v_cache8)) if fp8kv else (dev(w.k_cache), dev(w.v_cache))
        cq, sk, bt = i32(w.cu_seqlens_q), i32(w.seqlens_k), i32(w.block_table)
        o = torch.empty(w.q.shape, dtype=torch.float32, device="cuda")
        lse = torch.empty((w.hq, w.q.shape[0]), dtype=torch.float32, device="cuda")
        nseq = len(w.lengths_q)
        ws = t.paged_workspace(nseq, w.max_seqlen_q, w.max_seqlen_k, w.hq, w.hkv, w.d)
        call = t.attn_fwd_paged_fp8kv if fp8kv else t.attn_fwd_paged
        fn = lambda: call(q, kc, vc, cq, sk, bt, w.max_seqlen_q, w.max_seqlen_k,
                          scale=float(w.scale), causal=w.causal, out=o, lse=lse, workspace=ws)
        elem = 1 if fp8kv else 2
        by = (int(w.seqlens_k.sum()) * w.hkv * w.d * elem * 2 + w.q.size * 2 + w.q.size * 4
              + w.hq * w.q.shape[0] * 4)
        probe = time_calls(torch, fn, 3, 2)
        iters = int(min(30, max(5, 0.25e6 / max(1.0, statistics.median(probe)))))
        cold = time_calls(torch, fn, iters, 1, flush=flush)
        med = statistics.median(cold)
        gbs = by / (med * 1e-6) / 1e9
        # the same calls after a writing flush (its dirty lines drain during the call)
        wmed = statistics.median(time_calls(torch, fn, iters, 0, flush=flush.write))
        rows.append({"workload": name, "us_median_cold": round(med, 1),
                     "us_median_after_write_flush": round(wmed, 1), "mb": round(by / 1e6, 1),
                     "tokens_per_s": round(len(w.q) / (med * 1e-6), 1),
                     "gbs": round(gbs, 1), "pct_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 1),
                     "split_workspace_mb": round((ws.numel() if ws is not None else 0) / 1e6, 2)})
        del q, kc, vc, o, lse, ws, cq, sk, bt
        torch.cuda.empty_cache()
    return rows


def run_fp8(torch, t, names, flush):
    """attn_fwd_fp8_varlen per fp8 workload (cold cache); FLOPs as for bf16."""
    import numpy as np
    from synth import gen
    rows = []
    for name in names:
        w = gen.build_fp8(name)
        u8 = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda")
        q, k, v = u8(w.q), u8(w.k), u8(w.v)
        cq, ck = u8(w.cu_seqlens_q), u8(w.cu_seqlens_k)
        o = torch.empty(w.q.shape, dtype=torch.float32, device="cuda")
        lse = torch.empty((w.hq, w.q.shape[0]), dtype=torch.float32, device="cuda")
        fn = lambda: t.attn_fwd_fp8_varlen(q, k, v, cq, ck, w.max_seqlen, scale=float(w.scale),
                                           causal=w.causal, out=o, lse=lse)
        fl = 4.0 * w.d * w.hq * visible_pairs(w.lengths_q, w.lengths_k, w.causal)
        probe = time_calls(torch, fn, 3, 2)
        iters = int(min(30, max(5, 0.25e6 / max(1.0, statistics.median(probe)))))
        cold = time_calls(torch, fn, iters, 1, flush=flush)
        med = statistics.median(cold)
        tf = fl / (med * 1e-6) / 1e12
        rows.append({"workload": name, "us_median_cold": round(med, 1), "gflop": round(fl / 1e9, 2),
                     "tflops": round(tf, 1), "pct_fp8_peak": round(100 * tf / PEAK_FP8_TFLOPS, 1),
                     "pct_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 1)})
        del q, k, v, o, lse
        torch.cuda.empty_cache()
    return rows


# ------------------------------------------------------------------------- CPU baseline
def host_threads():
    """(host cores this process may use, BLAS threads NumPy's library runs)."""
    cores = len(os.sched_getaffinity(0))
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        blas = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        blas = cores
    return cores, blas


def oracle_config_time(w, budget_s=2.5):
    """Wall time of the fp64 oracle for one workload, from a bounded sample.

    The oracle works one (sequence, head) at a time (oracle.attention_one on
    that unit's decoded rows, the per-unit step of attention_varlen and
    attention_dense), materialising the full Lq x Lk score matrix.  Units are
    taken in a seeded random order until the budget is spent; the total is
    the sample's time scaled by (all units' Lq * Lk * (D + 1)) / (the sample's).
    Padded workloads add the oracle's gather and scatter of the whole input."""
    import numpy as np
    import oracle
    units = []
    if w.kind == "dense":
        for b in range(w.q.shape[0]):
            for h in range(w.hq):
                units.append((b, h))
    else:
        for s in range(len(w.lengths_q)):
            if w.lengths_q[s] > 0:
                for h in range(w.hq):
                    units.append((s, h))
    group = w.hq // w.hkv
    cost = lambda u: w.lengths_q[u[0]] * w.lengths_k[u[0]] * (w.d + 1)
    total_cost = sum(cost(u) for u in units)
    order = np.random.Generator(np.random.PCG64(99)).permutation(len(units))
    t_extra = 0.0
    if w.kind == "padded":
        t0 = time.perf_counter()
        hd = w.q.shape[2:]
        q, k, v = (oracle.unpad_gather(x, w.indices, hd) for x in (w.q, w.k, w.v))
        oracle.pad_scatter(np.zeros((len(w.indices),) + tuple(hd)), w.indices, w.q.shape[1])
        t_extra = time.perf_counter() - t0
    else:
        q, k, v = w.q, w.k, w.v
    cq, ck = w.cu_seqlens_q, w.cu_seqlens_k
    scale = np.float32(w.scale)
    done_cost, t_units, n = 0, 0.0, 0
    for i in order:
        s, h = units[i]
        g = h // group
        t0 = time.perf_counter()
        if w.kind == "dense":
            qs, ks, vs = q[s, :, h], k[s, :, g], v[s, :, g]
        else:
            qs, ks, vs = q[cq[s]:cq[s + 1], h], k[ck[s]:ck[s + 1], g], v[ck[s]:ck[s + 1], g]
        oracle.attention_one(oracle.bf16_bits_to_f64(qs), oracle.bf16_bits_to_f64(ks),
                             oracle.bf16_bits_to_f64(vs), scale, w.causal)
        t_units += time.perf_counter() - t0
        done_cost += cost(units[i])
        n += 1
        if t_units >= budget_s:
            break
    est = t_extra + t_units * total_cost / max(1, done_cost)
    full = n == len(units)
    return {"s": round(est, 3), "kind": "oracle",
            "sample": (f"all {n} (sequence, head) units" if full else
                       f"{n} of {len(units)} (sequence, head) units in {t_units:.2f} s, scaled by "
                       f"Lq*Lk*(D+1) to the whole workload (extrapolated)")
            + (", plus gather and scatter of the padded input" if w.kind == "padded" else "")}


def cpu_baseline(step_workloads, budget_s=20.0):
    """The fp64 oracle on the host, for the same padded-path step."""
    import numpy as np
    import oracle
    cores, threads = host_threads()
    flops = sum(attn_flops(w) for w in step_workloads)
    t0 = time.perf_counter()
    steps = 0
    while True:
        for w in step_workloads:
            hd = w.q.shape[2:]
            g = [oracle.unpad_gather(x, w.indices, hd) for x in (w.q, w.k, w.v)]
            o, _ = oracle.attention_varlen(*g, w.cu_seqlens_q, w.cu_seqlens_k, w.scale, True)
            oracle.pad_scatter(o, w.indices, w.q.shape[1])
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or steps >= 5:
            break
    per_step = el / steps
    return {"value": round(flops / per_step / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "host_cores": cores, "blas_threads": threads, "kind": "oracle",
            "sample": f"{steps} full step(s) of the same padded-path workload ((a) and (b)): NumPy fp64 "
                      f"gather, attention_varlen, scatter; {per_step * 1e3:.0f} ms per step"}


# ------------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--configs", default="all",
                    help="comma list of extra workloads to time per call, 'all' or 'none'")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--bwd-configs", default="varlen_1x8192,hdim_sweep_d128,hdim_sweep_d64,hdim_sweep_d32,hdim_sweep_d256",
                    help="comma list of workloads whose backward is timed, or 'none'")
    ap.add_argument("--paged-configs", default="all",
                    help="comma list of paged KV-cache workloads, 'all' or 'none'")
    ap.add_argument("--fp8-configs", default="all",
                    help="comma list of fp8 workloads, 'all' or 'none'")
    ap.add_argument("--only-configs", action="store_true",
                    help="time only the per-workload rows (no step, no JSON contract line)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path (the forward "
              "would shard by heads or sequences with no communication between GPUs).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import tiled_attention_fwd_amd as t
    from synth import gen

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    print(f"[bench] device {torch.cuda.get_device_name(0)}", file=sys.stderr, flush=True)

    if args.only_configs:
        flush = CacheFlush(torch)
        cfg_names = [] if args.configs == "none" else (
            list(gen.WORKLOADS) if args.configs == "all" else args.configs.split(","))
        for row in run_configs(torch, t, cfg_names, flush):
            print(json.dumps(row), flush=True)
        if args.bwd_configs != "none":
            for row in run_backward(torch, t, args.bwd_configs.split(","), flush):
                print(json.dumps({"backward": row}), flush=True)
        if args.paged_configs != "none":
            pn = list(gen.PAGED_WORKLOADS) if args.paged_configs == "all" else args.paged_configs.split(",")
            for row in run_paged(torch, t, pn, flush):
                print(json.dumps({"paged": row}), flush=True)
        if args.fp8_configs != "none":
            fn_ = list(gen.FP8_WORKLOADS) if args.fp8_configs == "all" else args.fp8_configs.split(",")
            for row in run_fp8(torch, t, fn_, flush):
                print(json.dumps({"fp8": row}), flush=True)
        return

    names = ["padded_32x128_random", "padded_1x2048"]
    wls = [gen.build_workload(n) for n in names]
    paths = [PaddedPath(w, torch, t) for w in wls]
    flops_step = sum(attn_flops(w) for w in wls)

    def busy():
        # ~1.5 ms of spinning: room for a batch of 20 launches to be enqueued
        for _ in range(3):
            spin(torch)

    def step():
        for p in paths:
            p.gather()
            p.attention()
            p.scatter()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # The step is captured once as a HIP graph so that host launch overhead
    # (the Python binding) does not starve the GPU between the six launches.
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)

    # Timed region 1: K graph replays back to back (wall clock -> value).
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = flops_step / (ms_per_step * 1e-3) / 1e12

    # The same replays cold: before each one a pass over 1 GiB evicts L2 and
    # MALL (outside the span); HIP events on the replay stream bracket the step.
    # Also after a writing pass, whose dirty lines drain during the step.
    flush = CacheFlush(torch)
    s_rep = torch.cuda.current_stream()

    def replay_after(fl):
        out = []
        for _ in range(max(5, min(args.steps, 50))):
            fl()
            ea = torch.cuda.Event(enable_timing=True)
            eb = torch.cuda.Event(enable_timing=True)
            ea.record(s_rep)
            graph.replay()
            eb.record(s_rep)
            eb.synchronize()
            out.append(ea.elapsed_time(eb) * 1e3)
        return out

    cold_us = replay_after(flush)
    step_cold_us = statistics.median(cold_us)
    step_wflush_us = statistics.median(replay_after(flush.write))

    # The fused padded path (attn_fwd_padded: zero fill + attention reading and
    # writing the padded rows) on the same inputs, captured and replayed alike.
    # Reported beside `value`, which stays on the three-call path.
    def fused_step():
        for p in paths:
            p.fused()

    gf = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        fused_step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(gf):
        fused_step()
    for _ in range(args.warmup):
        gf.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        gf.replay()
    torch.cuda.synchronize()
    ms_fused = (time.perf_counter() - t0) * 1e3 / args.steps
    fused_same = all(bool(torch.equal(p.out, p.out_f)) and bool(torch.equal(p.lse, p.lse_f))
                     for p in paths)

    # The same step with its two independent halves (the slot batch and the
    # long sequence) on two HIP streams, forked and joined inside one graph,
    # so the small latency-bound launches run beside the long attention.
    # Reported beside `value`, which stays on the one-stream step.
    outs_serial = [(p.out.clone(), p.lse.clone()) for p in paths]
    fork = torch.cuda.Stream()

    def concurrent_step():
        main = torch.cuda.current_stream()
        fork.wait_stream(main)
        paths[1].gather()
        paths[1].attention()
        paths[1].scatter()
        with torch.cuda.stream(fork):
            paths[0].gather()
            paths[0].attention()
            paths[0].scatter()
        main.wait_stream(fork)

    gc = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        concurrent_step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(gc):
        concurrent_step()
    for _ in range(args.warmup):
        gc.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        gc.replay()
    torch.cuda.synchronize()
    ms_conc = (time.perf_counter() - t0) * 1e3 / args.steps
    conc_same = all(bool(torch.equal(p.out, o)) and bool(torch.equal(p.lse, l))
                    for p, (o, l) in zip(paths, outs_serial))

    # Timed region 2: per-launch device time of each kernel of the step.  For
    # each launch kind, a spin kernel is queued first so the host can enqueue a
    # batch of identical launches (same inputs and outputs, so idempotent)
    # before the GPU reaches them; one pair of HIP events on the launch stream
    # brackets the batch, and the average per launch is elapsed / batch.
    s = torch.cuda.current_stream()
    kinds = [(pi, k) for pi in range(len(paths)) for k in ("gather", "attention", "scatter")]
    batch = 20
    avg_us = {}
    busy()  # first use of the spin kernel loads its code; keep that out of the timing
    torch.cuda.synchronize()
    for kk in kinds:
        pi, kname = kk
        fn = getattr(paths[pi], kname)
        samples = []
        for it in range(1 + max(1, args.steps // batch)):
            torch.cuda.synchronize()
            busy()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(s)
            for _ in range(batch):
                fn()
            b.record(s)
            b.synchronize()
            if it > 0:  # the first batch is an untimed warm-up
                samples.append(a.elapsed_time(b) * 1e3 / batch)
        avg_us[kk] = statistics.median(samples)
    print(f"[bench] {ms_per_step * 1e3:.1f} us/step (graph replay); per launch: " +
          ", ".join(f"{names[pi]}:{k}={v:.1f}us" for (pi, k), v in avg_us.items()),
          file=sys.stderr, flush=True)

    # Dominant kernel: the launch kind with the largest time per step.
    dom = max(avg_us, key=lambda kk: avg_us[kk])
    pi, kname = dom
    w, p = wls[pi], paths[pi]
    if kname == "attention":
        fl, by = attn_flops(w), attn_bytes(w)
        t_m, t_h = fl / (PEAK_BF16_TFLOPS * 1e12), by / (PEAK_HBM_GBS * 1e9)
        if t_m >= t_h:
            roof = {"bound": "mfma", "achieved": fl / (avg_us[dom] * 1e-6) / 1e12,
                    "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
        else:
            roof = {"bound": "hbm", "achieved": by / (avg_us[dom] * 1e-6) / 1e9,
                    "peak": PEAK_HBM_GBS, "unit": "GB/s"}
        tag = f"attn_fwd_{names[pi]}"
    else:
        by = p.bytes_gather() if kname == "gather" else p.bytes_scatter()
        roof = {"bound": "hbm", "achieved": by / (avg_us[dom] * 1e-6) / 1e9, "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
        tag = f"{kname}_{names[pi]}"
    roof["achieved"] = round(roof["achieved"], 2)
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = read_traffic(tag)
    roof["kernel"] = f"{kname} ({names[pi]})"
    roof["avg_launch_us"] = round(avg_us[dom], 2)

    cfg_rows = []
    if args.configs != "none":
        cfg_names = list(gen.WORKLOADS) if args.configs == "all" else args.configs.split(",")
        print(f"[bench] timing {len(cfg_names)} workloads", file=sys.stderr, flush=True)
        cfg_rows = run_configs(torch, t, cfg_names, flush, 0.0 if args.no_cpu else 2.5)
    bwd_rows = []
    if args.bwd_configs != "none":
        print("[bench] timing the backward", file=sys.stderr, flush=True)
        bwd_rows = run_backward(torch, t, args.bwd_configs.split(","), flush)
    paged_rows = []
    if args.paged_configs != "none":
        print("[bench] timing the paged KV-cache workloads", file=sys.stderr, flush=True)
        pn = list(gen.PAGED_WORKLOADS) if args.paged_configs == "all" else args.paged_configs.split(",")
        paged_rows = run_paged(torch, t, pn, flush)
    fp8_rows = []
    if args.fp8_configs != "none":
        print("[bench] timing the fp8 workloads", file=sys.stderr, flush=True)
        fn_ = list(gen.FP8_WORKLOADS) if args.fp8_configs == "all" else args.fp8_configs.split(",")
        fp8_rows = run_fp8(torch, t, fn_, flush)
    del flush

    cpu = None
    if not args.no_cpu:
        print("[bench] oracle CPU baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wls)

    line = {
        "metric": "fwd attention TFLOP/s & % bf16 MFMA peak; us/call varlen 32x64..1x8192",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"timing": "value: K replays of the step captured as a HIP graph; per_launch_us: HIP events around batches of 20 identical launches, queue pre-filled by a spin kernel", "workload": "packed LLM path with padding: B=1 total_len=4096 H=16 D=128 causal, "
                               "(a) 32 slots x 128 with valid lengths U{1..128} + (b) 1x2048 valid "
                               "+ 2048 padding; unpad gather -> varlen attention -> pad scatter",
                   "global_batch": 2, "seq_len": 4096, "parallelism": "none (1 GPU)",
                   "per_launch_us": {f"{names[pi]}:{k}": round(v, 2) for (pi, k), v in avg_us.items()},
                   "pct_bf16_peak_step": round(100 * value / PEAK_BF16_TFLOPS, 2),
                   "step_cold": {"timing": "one graph replay per sample, L2 and MALL evicted "
                                           "before each by a read pass over 1 GiB, HIP events "
                                           "around it",
                                 "us_median": round(step_cold_us, 2),
                                 "us_median_after_write_flush": round(step_wflush_us, 2),
                                 "us_p10": round(sorted(cold_us)[len(cold_us) // 10], 2),
                                 "us_p90": round(sorted(cold_us)[(len(cold_us) * 9) // 10], 2),
                                 "tflops": round(flops_step / (step_cold_us * 1e-6) / 1e12, 2)},
                   "fused_path": {"call": "attn_fwd_padded (zero fill + attention in place on "
                                          "the padded rows), same inputs and outputs",
                                  "ms_per_step": round(ms_fused, 4),
                                  "tflops": round(flops_step / (ms_fused * 1e-3) / 1e12, 2),
                                  "bitwise_equal_to_step": fused_same},
                   "two_stream_path": {"call": "the same six launches, the two halves on two "
                                               "HIP streams forked and joined in one graph",
                                       "ms_per_step": round(ms_conc, 4),
                                       "tflops": round(flops_step / (ms_conc * 1e-3) / 1e12, 2),
                                       "bitwise_equal_to_step": conc_same}},
        "roofline": roof,
        "cpu_baseline": cpu,
        "configs": cfg_rows,
        "backward": bwd_rows,
        "paged": paged_rows,
        "fp8": fp8_rows,
        "kernel_source_hash": source_hash(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
