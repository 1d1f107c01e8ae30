"""Helpers for the GPU tests: device detection, H2D/D2H of bf16 bit patterns,
and the element-wise / norm-wise comparisons against the oracle."""
from __future__ import annotations

import numpy as np

from rope_head_mixing_amd import synthetic

# Tolerances (stated once, used by every parity test):
#   bf16 outputs Y and dO: |gpu - ref| <= 1e-2 * |ref| + 1e-3, element-wise,
#       against the unrounded fp64 oracle value;
#   fp32 dW: ||gpu - ref||_F / ||ref||_F <= 1e-4, and every element within
#       1e-4 * max|ref|.
Y_RTOL, Y_ATOL = 1e-2, 1e-3
DW_REL = 1e-4


def has_gfx950() -> bool:
    try:
        import torch
    except ImportError:
        return False
    if not torch.cuda.is_available():
        return False
    name = getattr(torch.cuda.get_device_properties(0), "gcnArchName", "")
    return name.startswith("gfx950")


def dev_bf16(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def dev_i32(x: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def host_bits(t) -> np.ndarray:
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return synthetic.bf16_bits_to_f32(bits).astype(np.float64)


def check_bf16(gpu_bits: np.ndarray, ref: np.ndarray, label: str) -> float:
    """Element-wise bound; returns the worst |err| / bound ratio (must be <= 1)."""
    got = bf16_to_f64(gpu_bits)
    assert got.shape == ref.shape, (label, got.shape, ref.shape)
    err = np.abs(got - ref)
    bound = Y_RTOL * np.abs(ref) + Y_ATOL
    ratio = err / bound
    worst = float(ratio.max()) if ratio.size else 0.0
    if worst > 1.0:
        i = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
        raise AssertionError(f"{label}: {int((ratio > 1).sum())} of {ratio.size} elements out of "
                             f"tolerance; worst at {i}: gpu={got[i]!r} ref={ref[i]!r}")
    return worst


def check_dw(gpu: np.ndarray, ref: np.ndarray, label: str) -> float:
    gpu = np.asarray(gpu, np.float64)
    num = float(np.linalg.norm(gpu - ref))
    den = float(np.linalg.norm(ref))
    rel = num / den if den > 0 else num
    assert rel <= DW_REL, f"{label}: ||dW - ref||_F / ||ref||_F = {rel:.3e} > {DW_REL}"
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    worst = float(np.abs(gpu - ref).max()) if ref.size else 0.0
    assert worst <= DW_REL * max(scale, 1e-30), f"{label}: max |dW - ref| = {worst:.3e}"
    return rel
