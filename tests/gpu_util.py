"""Helpers shared by the GPU tests: device transfer and the parity bar."""

from __future__ import annotations

import numpy as np

# Parity bar for floating point outputs (bf16 inputs, fp32 outputs):
# max |O - O_ref| <= 2e-2, mean |O - O_ref| <= 2e-3, |LSE - LSE_ref| <= 1e-3.
O_MAX_ABS = 2e-2
O_MEAN_ABS = 2e-3
LSE_MAX_ABS = 1e-3


# Gradient bar (bf16 inputs, P and dS rounded to bf16 as MFMA operands, fp32
# accumulation): relative to the gradient's scale G = max(1, max |ref|),
# max |g - ref| <= 1e-2 G (about five bf16 unit roundoffs, 2^-9 each) and
# mean |g - ref| <= 1e-3 G (about half of one).
GRAD_MAX_REL = 1e-2
GRAD_MEAN_REL = 1e-3


def dev_bf16(bits: np.ndarray):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to("cuda").view(torch.bfloat16)


def dev_i32(x: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to("cuda")


def host(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def check_o(o_gpu: np.ndarray, o_ref: np.ndarray, what: str = "O") -> dict:
    assert o_gpu.shape == o_ref.shape, (o_gpu.shape, o_ref.shape)
    assert not np.isnan(o_gpu).any(), f"{what}: NaN in GPU output"
    err = np.abs(o_gpu.astype(np.float64) - o_ref)
    mx = float(err.max()) if err.size else 0.0
    mean = float(err.mean()) if err.size else 0.0
    assert mx <= O_MAX_ABS, f"{what}: max abs err {mx:.3e} > {O_MAX_ABS}"
    assert mean <= O_MEAN_ABS, f"{what}: mean abs err {mean:.3e} > {O_MEAN_ABS}"
    return {"max": mx, "mean": mean}


def check_lse(l_gpu: np.ndarray, l_ref: np.ndarray, what: str = "LSE") -> float:
    assert l_gpu.shape == l_ref.shape, (l_gpu.shape, l_ref.shape)
    assert not np.isnan(l_gpu).any(), f"{what}: NaN"
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(l_gpu), fin), f"{what}: finiteness differs"
    assert np.array_equal(l_gpu[~fin], l_ref[~fin].astype(np.float32)), f"{what}: -inf rows differ"
    if not fin.any():
        return 0.0
    e = float(np.abs(l_gpu[fin].astype(np.float64) - l_ref[fin]).max())
    assert e <= LSE_MAX_ABS, f"{what}: max abs err {e:.3e} > {LSE_MAX_ABS}"
    return e


def check_grad(g_gpu: np.ndarray, g_ref: np.ndarray, what: str) -> dict:
    assert g_gpu.shape == g_ref.shape, (g_gpu.shape, g_ref.shape)
    assert np.isfinite(g_gpu).all(), f"{what}: non-finite value in GPU gradient"
    if g_ref.size == 0:
        return {"max": 0.0, "mean": 0.0, "scale": 0.0}
    scale = max(1.0, float(np.abs(g_ref).max()))
    err = np.abs(g_gpu.astype(np.float64) - g_ref)
    mx, mean = float(err.max()), float(err.mean())
    assert mx <= GRAD_MAX_REL * scale, f"{what}: max abs err {mx:.3e} > {GRAD_MAX_REL} * {scale:.3g}"
    assert mean <= GRAD_MEAN_REL * scale, f"{what}: mean abs err {mean:.3e} > {GRAD_MEAN_REL} * {scale:.3g}"
    return {"max": mx, "mean": mean, "scale": scale}
