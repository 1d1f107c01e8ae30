"""Seeded random shapes through every route of the gfx950 path, against the
fp64 oracle.

The hand-picked cases of test_parity_gpu.py aim at one route each; this sweep
draws head counts from 1 to 128 (padded rows, several tokens per tile, 96- and
128-row tiles), channel splits with and without d a multiple of 128 (tiled and
general kernels), pe from 0 to 256 and short ragged token counts, and eight
more with 1100 to 4000 tokens, where the token blocks are rounded to whole
rounds and spread evenly, and forty more drawn per head-count band with
rows up to 1280 channels.  Each shape
runs the forward, dx, dW and the single-call backward, each checked against
the oracle, and the single-call dO must equal postmix_bwd_dx's bit for bit.
Head counts start at one: a single dW entry may cancel to far below the sum
of its terms' magnitudes, which the dW bound's u * A term (tests/gpu_util.py)
accounts for.
"""
import numpy as np
import pytest

import oracle
from rope_head_mixing_amd import synthetic
from tests import gpu_util as gu
from tests.test_parity_gpu import Dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gu.has_gfx950(), reason="needs an MI355X (gfx950)")]


def _shapes(n: int, seed: int = 20261202):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        nh = int(rng.integers(1, 129))
        if rng.random() < 0.6:  # d a multiple of 128: the tiled kernels
            d = int(rng.choice([128, 256, 384, 512, 640]))
            pe = 16 * int(rng.integers(0, min(d, 256) // 16 + 1))
        else:
            d = 8 * int(rng.integers(1, 80))
            pe = 16 * int(rng.integers(0, min(d, 256) // 16 + 1))
        nope = d - pe
        sq = int(rng.integers(1, 61 if nh <= 64 else 21))
        off = int(rng.integers(0, 30000))
        out.append((sq, nh, nope, pe, off))
    return out


SHAPES = _shapes(120)


@pytest.mark.parametrize("sq,nh,nope,pe,off", SHAPES)
def test_random_shape(sq, nh, nope, pe, off):
    c = synthetic.case(sq, nh, nope, pe, seed=7000 + 13 * sq + nh, pos_offset=off)
    print(f"\n[parity] random {c.name} off={off}", flush=True)
    dv = Dev(c)
    Y = gu.host_bits(dv.fwd())
    gu.check_bf16(Y, oracle.fwd(dv.O, dv.W, dv.pos, c.theta, nope, pe), f"{c.name} Y")
    dO_dx = gu.host_bits(dv.dx())
    ref_dO = oracle.bwd_dx(dv.dY, dv.W, dv.pos, c.theta, nope, pe)
    gu.check_bf16(dO_dx, ref_dO, f"{c.name} dO")
    ref_dW, mag = gu.dw_refs(dv.dY, dv.O, dv.pos, c.theta, nope, pe)
    gu.check_dw(dv.dw().cpu().numpy(), ref_dW, f"{c.name} dW", mag)
    dO, dW = dv.bwd()
    np.testing.assert_array_equal(gu.host_bits(dO), dO_dx)
    gu.check_dw(dW.cpu().numpy(), ref_dW, f"{c.name} bwd dW", mag)


def _large_shapes(n: int, seed: int = 20261203):
    """Token counts large enough that the token blocks are rounded to whole
    rounds and spread evenly (more than 256 blocks of the fused backward, and
    of the weight gradient above 64 heads); d = 128 or 256 keeps the oracle
    at seconds."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        nh = int(rng.integers(1, 129))
        d = int(rng.choice([128, 256]))
        pe = int(rng.choice([0, 32, 64]))
        sq = int(rng.integers(1100, 1700)) if nh > 32 else int(rng.integers(2100, 4000))
        out.append((sq, nh, d - pe, pe, int(rng.integers(0, 30000))))
    return out


@pytest.mark.parametrize("sq,nh,nope,pe,off", _large_shapes(8))
def test_random_shape_many_blocks(sq, nh, nope, pe, off):
    test_random_shape(sq, nh, nope, pe, off)


def _banded_shapes(per_band: int = 8, seed: int = 20261204):
    """Eight shapes in each head-count band ([1, 4] fp32 small-head kernels,
    [5, 32] token-packed tiles, [33, 64], [65, 96], [97, 128]), with rows up
    to 1280 channels: nope a multiple of 8 in [0, 1024], pe a multiple of 16
    in [0, 256] (nope + pe > 0), sq in [1, 64], positions offset by [0, 40000)."""
    rng = np.random.default_rng(seed)
    out = []
    for lo, hi in [(1, 4), (5, 32), (33, 64), (65, 96), (97, 128)]:
        for _ in range(per_band):
            nh = int(rng.integers(lo, hi + 1))
            while True:
                nope = 8 * int(rng.integers(0, 129))
                pe = 16 * int(rng.integers(0, 17))
                if nope + pe > 0:
                    break
            out.append((int(rng.integers(1, 65)), nh, nope, pe, int(rng.integers(0, 40000))))
    return out


@pytest.mark.parametrize("sq,nh,nope,pe,off", _banded_shapes())
def test_banded_random_shape(sq, nh, nope, pe, off):
    test_random_shape(sq, nh, nope, pe, off)
