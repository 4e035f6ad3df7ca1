"""Builds libattnfwd.so (gfx950) in-tree with hipcc.

Usage: python -m tiled_attention_fwd_amd.build   (or call build()).
Objects go to tiled_attention_fwd_amd/_build/, the library next to this file.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libattnfwd.so")
MICROBENCH = os.path.join(PKG, "microbench")  # bench-only executable (unit rates, copy bandwidth)
SOURCES = ["attn_kernel.hip", "attn_kernel_d256.hip", "attn_bwd.hip", "decode_kernel.hip", "fp8_kernel.hip", "rows_kernel.hip", "debug_checks.hip", "noalloc.hip", "abi.cpp"]
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU ops.
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wno-unused-command-line-argument",
]


# Per-source flags.  Forward kernels that need more than 256 registers (head
# dim 256, one wave per SIMD) would otherwise get MFMA accumulators in AGPRs,
# and every score then costs a copy back to a VGPR for the softmax; VGPR-form
# MFMAs keep scores and outputs in VGPRs and spill only a few long-lived
# operands (head_dim 256 DMA kernel: ~900 -> ~50 AGPR copies per two tiles).
# The backward takes them too: its fused dK/dV pass at head_dim 128 then
# writes K and V once into AGPRs (MFMAs read them as operands there), which
# leaves the VGPRs to dK, dV and the S/dP blocks (80 -> 8 AGPR reads per query
# tile); gradients bit-identical, 1x8192 causal 1256 -> 1229 us, head_dim 256
# (two passes) 812 -> 734 us.  Without the K/V move the accumulators spilled
# and the pass was slower (1x8192: 1357 vs 1468 us).  The fp8 forward too: at
# head_dim 256 it then fits 256 registers (two waves per SIMD instead of one;
# 1 x 4096 causal 139 -> 108 us, bit-identical; other head dims unchanged).
# And the paged decode: at head_dim 256 it no longer spills to scratch (32
# sequences of 4-8k keys, 234 -> 112 us; E4M3 caches 64.6 -> 61.0 us).
# The iterative ILP scheduler places LDS reads further ahead of the MFMAs
# that use them, which pays where one wave per SIMD has to hide its own
# latencies: the head_dim 256 forward kernels (their own unit, 1 x 4096
# causal 212 -> 183 us) and the backward (dK/dV pass at one wave per SIMD;
# 1x8192 causal 1353 -> 1250 us).  The other forward kernels, fp8 and the
# paged decode measured within +-2 % with it and keep the default.
_VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
_ILP = ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]
EXTRA_FLAGS = {"attn_kernel.hip": _VGPR_FORM, "attn_kernel_d256.hip": _VGPR_FORM + _ILP,
               "attn_bwd.hip": _VGPR_FORM + _ILP, "fp8_kernel.hip": _VGPR_FORM,
               "decode_kernel.hip": _VGPR_FORM}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; a ROCm toolchain is required to build libattnfwd.so")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, *EXTRA_FLAGS.get(src, []), "-x", "hip", "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compiles every source and links the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    cmd = [hipcc(), *COMMON_FLAGS, "-x", "hip", os.path.join(CSRC, "microbench.hip"), "-o",
           MICROBENCH + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for microbench.hip:\n{r.stdout}\n{r.stderr}")
    os.replace(MICROBENCH + ".tmp", MICROBENCH)
    if verbose:
        print(f"built {LIB} and {MICROBENCH}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
