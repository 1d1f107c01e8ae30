"""Helpers for the GPU tests: device detection, H2D/D2H of bf16 bit patterns,
and the element-wise / norm-wise comparisons against the oracle."""
from __future__ import annotations

import numpy as np

from rope_head_mixing_amd import synthetic

# Tolerances (stated once, used by every parity test):
#   bf16 outputs Y and dO: |gpu - ref| <= 1e-2 * |ref| + 1e-3, element-wise,
#       against the unrounded fp64 oracle value;
#   fp32 dW: ||gpu - ref||_F <= 1e-4 * ||ref||_F + u * ||A||_F, and every
#       element |gpu - ref| <= 1e-4 * max|ref| + u * A[g,h], where
#       A[g,h] = sum |dY[s,g,c] * inv_rope(O)[s,h,c]| (oracle.bwd_dw_abs) and
#       u = 2^-24.  The u * A term is one fp32 rounding at the largest
#       magnitude a partial sum of the entry's terms can reach: it admits
#       entries that cancel to far below their terms (a single head's sum can
#       cancel to 6e-5 of them), and is negligible beside 1e-4 * max|ref| for
#       entries that do not.  Without A the bound is the relative one alone.
Y_RTOL, Y_ATOL = 1e-2, 1e-3
DW_REL = 1e-4
U32 = 2.0 ** -24


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


def check_dw(gpu: np.ndarray, ref: np.ndarray, label: str, mag: np.ndarray | None = None) -> float:
    """Norm-wise and element-wise dW bound (above); returns ||gpu - ref||_F / ||ref||_F."""
    gpu = np.asarray(gpu, np.float64)
    assert gpu.shape == ref.shape, (label, gpu.shape, ref.shape)
    err = np.abs(gpu - ref)
    num = float(np.linalg.norm(err))
    den = float(np.linalg.norm(ref))
    rel = num / den if den > 0 else num
    cond = 0.0 if mag is None else U32 * float(np.linalg.norm(mag))
    assert num <= DW_REL * den + cond, (f"{label}: ||dW - ref||_F = {num:.3e} > 1e-4 * {den:.3e}"
                                         f" + u * ||A||_F = {DW_REL * den + cond:.3e}")
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    bound = DW_REL * max(scale, 1e-30) + (0.0 if mag is None else U32 * np.asarray(mag, np.float64))
    bad = err > bound
    if np.any(bad):
        i = np.unravel_index(int(np.argmax(err - bound)), err.shape)
        raise AssertionError(f"{label}: {int(bad.sum())} dW entries out of bound; worst at {i}: "
                             f"gpu={gpu[i]!r} ref={ref[i]!r} bound={np.broadcast_to(bound, err.shape)[i]:.3e}")
    return rel


def dw_refs(dY, O, pos, theta, nope, pe):
    """(dW, A): the oracle's weight gradient and its terms' magnitude sums."""
    import oracle
    return (oracle.bwd_dw(dY, O, pos, theta, nope, pe),
            oracle.bwd_dw_abs(dY, O, pos, theta, nope, pe))


def check_bf16_streamed(gpu_bits: np.ndarray, ref_fn, label: str, chunk: int = 512,
                        progress_every: int = 8) -> float:
    """Element-wise bf16 bound over a whole [sq, nh, d] output, the fp64
    reference computed `chunk` tokens at a time by ref_fn(s0, s1) (so no fp64
    copy of the whole tensor is held).  Returns the worst |err| / bound."""
    sq = gpu_bits.shape[0]
    worst = 0.0
    n_chunks = (sq + chunk - 1) // chunk
    for j, s0 in enumerate(range(0, sq, chunk)):
        s1 = min(sq, s0 + chunk)
        worst = max(worst, check_bf16(gpu_bits[s0:s1], ref_fn(s0, s1), f"{label} tokens {s0}..{s1 - 1}"))
        if progress_every and (j + 1) % progress_every == 0:
            print(f"    {label}: {j + 1}/{n_chunks} chunks, worst err/bound {worst:.3f}", flush=True)
    return worst
