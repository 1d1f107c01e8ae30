"""Seeded synthetic inputs shared by the HIP path's tests/benchmark and the oracle.

This module holds no arithmetic of the method: it draws Gaussian tensors with
numpy's ``default_rng``, rounds them to bfloat16 (round-to-nearest-even) and
hands out the raw bf16 bit patterns (``uint16``) so that the GPU and the CPU
oracle see identical bytes.

Workloads follow the shapes of the production path measured in PaddleFleet
PR #1772 ("Fuse HCA inverse RoPE into the VHA postmix, ..."), PR body item 1:
sq=16384 tokens per context-parallel rank (64K context, CP=4), nh=64 heads,
nope=448 + pe=64 channels, a 1 GiB attention output.  Values are synthetic:
O and dY ~ N(0,1), W = I + N(0, 0.02), rotate-half RoPE with theta=10000.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

THETA = 10000.0


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits.

    Inputs are finite Gaussian draws, so NaN/Inf handling is not needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(seed: int, shape, scale: float = 1.0, rows_per_chunk: int = 1024) -> np.ndarray:
    """N(0, scale^2) draws (float32) rounded to bf16 bits, generated in row chunks."""
    rng = np.random.default_rng(seed)
    shape = tuple(int(v) for v in shape)
    out = np.empty(shape, np.uint16)
    if len(shape) == 0 or shape[0] == 0:
        return out
    flat = out.reshape(shape[0], -1)
    for r0 in range(0, shape[0], rows_per_chunk):
        r1 = min(shape[0], r0 + rows_per_chunk)
        v = rng.standard_normal((r1 - r0, flat.shape[1]), dtype=np.float32)
        if scale != 1.0:
            v *= np.float32(scale)
        flat[r0:r1] = f32_to_bf16_bits(v)
    return out


def postmix_weight(seed: int, nh: int, sigma: float = 0.02) -> np.ndarray:
    """W = I + N(0, sigma^2), rounded to bf16 bits, shape [nh, nh]."""
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((nh, nh), dtype=np.float32) * np.float32(sigma)
    v += np.eye(nh, dtype=np.float32)
    return f32_to_bf16_bits(v)


@dataclass
class Case:
    name: str
    sq: int
    nh: int
    nope: int
    pe: int
    pos_offset: int
    seeds: tuple  # (O, W, dY); dY seed None => forward only
    theta: float = THETA

    @property
    def d(self) -> int:
        return self.nope + self.pe

    def positions(self) -> np.ndarray:
        return (self.pos_offset + np.arange(self.sq, dtype=np.int64)).astype(np.int32)

    def O(self) -> np.ndarray:
        return normal_bf16(self.seeds[0], (self.sq, self.nh, self.d))

    def W(self) -> np.ndarray:
        return postmix_weight(self.seeds[1], self.nh)

    def dY(self) -> np.ndarray:
        seed = self.seeds[2] if self.seeds[2] is not None else self.seeds[0] + 2
        return normal_bf16(seed, (self.sq, self.nh, self.d))

    def algorithmic_bytes(self, op: str) -> int:
        """Bytes an op must move: activations in/out, W, touched cos/sin rows, positions, dW."""
        act = self.sq * self.nh * self.d * 2
        tables = self.sq * (self.pe // 2) * 4 * 2
        pos = self.sq * 4
        w = self.nh * self.nh * 2
        if op in ("fwd", "bwd_dx"):
            return 2 * act + w + tables + pos
        if op == "bwd_dw":
            return 2 * act + tables + pos + self.nh * self.nh * 4
        if op == "bwd":  # both gradients from one read of dY and O
            return 3 * act + w + tables + pos + self.nh * self.nh * 4
        raise ValueError(op)

    def flops(self) -> int:
        return 2 * self.nh * self.nh * self.sq * self.d


# The five workloads (tiny, forward-only, production forward, production
# backward, head-count sweep) with the seeds used throughout, and two more
# head counts for the 96-row kernels.
CASES = {
    "tiny": Case("tiny", 64, 4, 48, 16, 0, (1001, 1002, 1003)),
    "fwd_1k": Case("fwd_1k", 1024, 64, 448, 64, 0, (2001, 2002, None)),
    "prod": Case("prod", 16384, 64, 448, 64, 16384, (3001, 3002, 3003)),
    "sweep_nh3": Case("sweep_nh3", 8192, 3, 448, 64, 0, (5001, 5002, 5003)),
    "sweep_nh128": Case("sweep_nh128", 8192, 128, 448, 64, 0, (5011, 5012, 5013)),
    # head counts between 64 and 128 (96-row tiles and chunks), same recipe
    "sweep_nh96": Case("sweep_nh96", 8192, 96, 448, 64, 0, (5021, 5022, 5023)),
    "sweep_nh72": Case("sweep_nh72", 8192, 72, 448, 64, 0, (5031, 5032, 5033)),
}


def case(sq: int, nh: int, nope: int, pe: int, seed: int, pos_offset: int = 0,
         theta: float = THETA, name: str | None = None) -> Case:
    """An ad hoc case with seeds (seed, seed+1, seed+2)."""
    return Case(name or f"sq{sq}_nh{nh}_{nope}+{pe}", sq, nh, nope, pe, pos_offset,
                (seed, seed + 1, seed + 2), theta)
