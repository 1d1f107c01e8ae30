"""Parity of the gfx950 path (through the C ABI) with the fp64 oracle.

Tolerances (tests/gpu_util.py): bf16 Y and dO within 1e-2*|ref| + 1e-3 of the
fp64 oracle element by element; fp32 dW within 1e-4 relative (Frobenius norm,
and every element within 1e-4 * max|ref|), plus one fp32 rounding of the
entry's term magnitudes for entries that cancel; dW bitwise identical across
runs.

Inputs are the seeded synthetic workloads of rope_head_mixing_amd.synthetic:
the tiny case (sq=64, nh=4, 48+16), the forward-only case (sq=1024, nh=64,
448+64) and the nh = 3 head-count sweep (sq=8192); plus small shapes that
span several tiles with ragged tails.  The full-size workloads are compared
element by element in test_fullsize_gpu.py.
"""
import numpy as np
import pytest

import oracle
from rope_head_mixing_amd import synthetic
from tests import gpu_util as gu

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gu.has_gfx950(), reason="needs an MI355X (gfx950)")]

THETA = synthetic.THETA


def P():
    from rope_head_mixing_amd import postmix
    return postmix


def tables(case, positions):
    if case.pe == 0:
        return None, None
    rows = int(np.max(positions)) + 1 if len(positions) else 1
    return P().postmix_rope_table(case.theta, case.pe, rows)


class Dev:
    """Device copies of one case's inputs."""

    def __init__(self, case, O=None, W=None, dY=None, positions=None, need_dy=True):
        self.case = case
        self.O = case.O() if O is None else O
        self.W = case.W() if W is None else W
        self.dY = (case.dY() if dY is None else dY) if need_dy else None
        self.pos = case.positions() if positions is None else np.asarray(positions, np.int32)
        self.dO_ = gu.dev_bf16(self.O)
        self.dW_ = gu.dev_bf16(self.W)
        self.ddY_ = gu.dev_bf16(self.dY) if need_dy else None
        self.dpos = gu.dev_i32(self.pos)
        self.cos, self.sin = tables(case, self.pos)

    def fwd(self):
        c = self.case
        return P().postmix_fwd(self.dO_, self.dW_, self.cos, self.sin, self.dpos, c.nope, c.pe)

    def dx(self):
        c = self.case
        return P().postmix_bwd_dx(self.ddY_, self.dW_, self.cos, self.sin, self.dpos, c.nope, c.pe)

    def bwd(self, workspace=None):
        c = self.case
        return P().postmix_bwd(self.ddY_, self.dO_, self.dW_, self.cos, self.sin, self.dpos, c.nope,
                               c.pe, workspace=workspace)

    def dw(self, workspace=None):
        c = self.case
        return P().postmix_bwd_dw(self.ddY_, self.dO_, self.cos, self.sin, self.dpos, c.nope, c.pe,
                                  workspace=workspace)


def full_check(case, ops=("fwd", "dx", "dw")):
    """Every element of each op's output against the oracle.  "bwd" (the
    single-call backward) also needs "dx": its dO must be bitwise dx's."""
    print(f"\n[parity] {case.name}: sq={case.sq} nh={case.nh} nope={case.nope} pe={case.pe}",
          flush=True)
    dv = Dev(case, need_dy=any(op in ops for op in ("dx", "dw", "bwd")))
    out = {}
    if "fwd" in ops:
        Y = gu.host_bits(dv.fwd())
        ref = oracle.fwd(dv.O, dv.W, dv.pos, case.theta, case.nope, case.pe)
        out["fwd"] = gu.check_bf16(Y, ref, f"{case.name} Y")
    if "dx" in ops:
        dO = gu.host_bits(dv.dx())
        ref = oracle.bwd_dx(dv.dY, dv.W, dv.pos, case.theta, case.nope, case.pe)
        out["dx"] = gu.check_bf16(dO, ref, f"{case.name} dO")
    if "dw" in ops or "bwd" in ops:
        ref, mag = gu.dw_refs(dv.dY, dv.O, dv.pos, case.theta, case.nope, case.pe)
    if "dw" in ops:
        out["dw"] = gu.check_dw(dv.dw().cpu().numpy(), ref, f"{case.name} dW", mag)
    if "bwd" in ops:
        dO_f, dW_f = dv.bwd()
        np.testing.assert_array_equal(gu.host_bits(dO_f), dO)
        out["bwd_dw"] = gu.check_dw(dW_f.cpu().numpy(), ref, f"{case.name} fused dW", mag)
    print(f"[parity] {case.name}: {out}", flush=True)
    return out


# --------------------------------------------------------------------------
# first: the smallest launch, so a stall at compile/load time is told apart
# from a problem of volume
# --------------------------------------------------------------------------

def test_00_one_token_one_head():
    full_check(synthetic.case(1, 1, 0, 16, seed=7, pos_offset=3))


def test_01_rope_table_matches_oracle_angles():
    for pe, rows in [(16, 64), (64, 32768)]:
        cos, sin = P().postmix_rope_table(THETA, pe, rows)
        C, S = oracle.rope_angles(THETA, pe, np.arange(rows, dtype=np.int32))
        # fp32 rounding of values in [-1, 1]: at most 2^-25 from the fp64 value
        assert np.abs(cos.cpu().numpy().astype(np.float64) - C).max() <= 2.0 ** -24
        assert np.abs(sin.cpu().numpy().astype(np.float64) - S).max() <= 2.0 ** -24


def test_02_tiny_workload():
    full_check(synthetic.CASES["tiny"])


@pytest.fixture(params=["tiled", "general"])
def kernel_policy(request):
    """Run a test with the default (tiled where the shape allows) kernels, and
    again with every shape forced onto the general kernels."""
    prev = P().testing_set_general_kernels(request.param == "general")
    yield request.param
    P().testing_set_general_kernels(prev)


@pytest.mark.parametrize("sq,nh,nope,pe,off", [
    (128, 4, 48, 16, 0),       # the (128, 4, 64) shape the pages' tests single out
    (67, 64, 448, 64, 16384),  # production widths, ragged token count
    (33, 20, 40, 16, 5),       # nh not a multiple of 16, nope % 16 == 8
    (50, 3, 448, 64, 0),       # the smallest head count of the sweep
    (19, 128, 448, 64, 8000),  # widest head mix
    (40, 64, 512, 0, 0),       # pe = 0: plain head mix
    (40, 8, 0, 64, 1000),      # nope = 0: every channel rotated
    (21, 33, 8, 32, 77),       # nh just past a 32-head block
    (9, 96, 64, 16, 31),       # nh = 96 (three 32-head output blocks)
    (5, 1, 8, 16, 2),          # a single head
    (25, 32, 192, 64, 9),      # nh = 32, one 256-channel part
    (11, 64, 320, 64, 500),    # d = 384: 128-channel parts
    (7, 64, 384, 128, 3),      # pe = 128
    (13, 64, 432, 80, 4000),   # nope not a multiple of 32: an M-block straddles nope
    (6, 128, 192, 64, 17),     # nh = 128 with two 128-channel parts
    (3, 64, 0, 256, 100),      # every channel rotated, pe = one whole part
    (11, 64, 480, 32, 5),      # pe = 32: one paired pe block (partners 16 apart)
    (9, 64, 416, 96, 11),      # pe = 96: three paired pe blocks
    (8, 64, 464, 48, 21),      # nope % 32 != 0: pe rotated through the fp32 scratch
    (7, 128, 320, 64, 9),      # nh = 128, d = 384: 128-channel parts, heads split over wave groups
    (3, 128, 16, 240, 5),      # nh = 128 with an fp32 scratch too large for the LDS: general kernel
    (13, 20, 448, 64, 7),      # nh = 20: head rows padded to 32
    (5, 7, 448, 64, 2),        # nh = 7: padded to 32
    (9, 80, 448, 64, 3),       # nh = 80: padded to 96 (three wave groups)
    (7, 72, 192, 64, 11),      # nh = 72, d = 256: padded to 96
    (6, 96, 448, 64, 4000),    # nh = 96: 96-row tiles
    (37, 8, 448, 64, 3),       # nh = 8: four tokens per 32-row tile, last tile one token
    (23, 12, 192, 64, 9),      # nh = 12: two tokens per tile, d = 256
    (19, 16, 432, 80, 5),      # nh = 16: two tokens per tile, pe through the fp32 scratch
    (14, 5, 448, 64, 1),       # nh = 5: six tokens per tile (30 of 32 rows)
    (17, 5, 320, 64, 11),      # nh = 5, d = 384: 128-channel parts
    (9, 5, 256, 128, 4),       # nh = 5, pe = 128 in 128-channel parts
    (7, 6, 0, 256, 3),         # nh = 6, every channel rotated: five tokens' cos/sin rows
    (21, 8, 512, 0, 0),        # nh = 8, pe = 0
    (70, 2, 192, 64, 5),       # nh = 2: 32 tokens per 64-row tile, ragged last tile
    (40, 3, 320, 64, 1),       # nh = 3, 128-channel parts: the angle rows cap the tile at 16 tokens
    (45, 1, 448, 64, 3),       # nh = 1: 32 tokens per 32-row tile
    (29, 12, 448, 64, 8),      # nh = 12: five tokens per 64-row tile
    (33, 32, 448, 64, 2),      # nh = 32: exact 32-row mix tiles, two tokens per weight-gradient chunk
])
def test_small_shapes(sq, nh, nope, pe, off, kernel_policy):
    full_check(synthetic.case(sq, nh, nope, pe, seed=1000 + sq + nh, pos_offset=off))


@pytest.mark.parametrize("sq,nh,nope,pe", [(70, 64, 448, 64), (21, 128, 448, 64), (30, 32, 432, 80)])
def test_tiled_and_general_kernels_agree(sq, nh, nope, pe):
    """Both kernel families on the same inputs: the MFMA inputs and k order are
    the same, so nope outputs agree bitwise; rotated outputs may differ by the
    fp32 evaluation order of the rotation (one bf16 ulp at most)."""
    c = synthetic.case(sq, nh, nope, pe, seed=777, pos_offset=16384)
    dv = Dev(c)
    prev = P().testing_set_general_kernels(False)
    try:
        Y1, dO1, dW1 = gu.host_bits(dv.fwd()), gu.host_bits(dv.dx()), dv.dw().cpu().numpy()
        P().testing_set_general_kernels(True)
        Y2, dO2, dW2 = gu.host_bits(dv.fwd()), gu.host_bits(dv.dx()), dv.dw().cpu().numpy()
    finally:
        P().testing_set_general_kernels(prev)
    np.testing.assert_array_equal(Y1[..., :nope], Y2[..., :nope])
    np.testing.assert_array_equal(dO1[..., :nope], dO2[..., :nope])
    for a, b in [(Y1, Y2), (dO1, dO2)]:
        fa, fb = gu.bf16_to_f64(a[..., nope:]), gu.bf16_to_f64(b[..., nope:])
        # one bf16 ulp is at most 2^-7 of the value
        assert np.all(np.abs(fa - fb) <= 2.0 ** -7 * np.abs(fb) + 1e-30), \
            "rotated outputs differ by more than one bf16 ulp"
    rel = np.linalg.norm(dW1 - dW2) / np.linalg.norm(dW2)
    assert rel < 1e-5, rel


@pytest.mark.parametrize("sq,nh,nope,pe,off", [
    (67, 64, 448, 64, 16384),   # fused path, ragged block count
    (33, 64, 192, 64, 7),       # fused path, d = 256
    (70, 64, 384, 128, 3),      # fused path, pe = 128 (one whole chunk rotated)
    (19, 64, 432, 80, 99),      # fused path, nope straddles an M-block
    (13, 64, 480, 32, 7),       # fused path, pe = 32 (one paired pe block)
    (9, 64, 416, 96, 11),       # fused path, pe = 96 (three paired pe blocks)
    (11, 64, 496, 16, 5),       # fused path, pe = 16 (fp32 scratch)
    (13, 128, 448, 64, 5),      # fused path, nh = 128 (waves split by gradient)
    (9, 128, 192, 64, 3),       # fused path, nh = 128, d = 256
    (7, 128, 384, 128, 11),     # fused path, nh = 128, pe = 128
    (5, 128, 432, 80, 2),       # not fused (nh = 128 with pe = 80): separate kernels
    (11, 48, 448, 64, 3),       # fused path, nh = 48 (head rows padded to 64)
    (9, 33, 192, 64, 1),        # fused path, nh = 33, d = 256
    (7, 96, 448, 64, 5),        # fused path, nh = 96: 96-row chunks of 256 channels on 12 waves
    (9, 72, 448, 64, 3),        # fused path, nh = 72: 96-row chunks, rows 72..95 padding
    (11, 65, 192, 64, 2),       # fused path, nh = 65, d = 256: 96-row chunks, one real row in the last N-block
    (8, 80, 224, 32, 4),        # fused path, nh = 80, pe = 32 (one paired pe block), 96-row chunks
    (6, 96, 256, 0, 1),         # fused path, nh = 96, no pe
    (5, 96, 384, 128, 7),       # fused path, nh = 96, pe = 128: the 96-row LDS does not fit, 128-row chunks
    (7, 90, 320, 64, 1),        # fused path, nh = 90, d = 384 (not a multiple of 256): 128-row chunks
    (520, 72, 448, 64, 9),      # fused path, nh = 72: 260 blocks of 2 tokens -> 256 blocks
    (6, 100, 432, 80, 9),       # not fused (padded to 128 with pe = 80): separate kernels
    (21, 32, 448, 64, 5),       # fused path, nh = 32: two tokens per 64-row chunk
    (9, 3, 448, 64, 0),         # fused path, nh = 3: one partial chunk of 9 of 21 tokens
    (300, 3, 448, 64, 7),       # fused path, nh = 3: 15 blocks of 21 tokens, the last one partial
    (37, 8, 192, 64, 2),        # fused path, nh = 8, d = 256: eight tokens per chunk
    (29, 5, 320, 64, 3),        # fused path, nh = 5, d = 384: 128-channel chunks, 12 tokens each
    (23, 20, 496, 16, 9),       # fused path, nh = 20, pe = 16: pe through the fp32 scratch
    (41, 1, 448, 64, 11),       # fused path, nh = 1: 32 tokens per chunk (the cos/sin group)
    (40, 1, 448, 64, 11),       # the same at sq = 40: with this seed the single dW entry cancels
                                # to 6e-5 of the sum of its terms' magnitudes (the bound's u * A term)
    (12, 1, 496, 16, 1),        # not fused (nh = 1, pe = 16: 64 tokens would exceed the cos/sin group)
    # block counts rounded to a multiple of 256, token groups spread evenly
    (2400, 8, 192, 64, 3),      # 300 blocks of one 8-token chunk -> 256 blocks of 1 or 2 chunks
    (4800, 64, 192, 64, 11),    # 600 blocks of 8 tokens -> 512 blocks of 9 or 10
    (1200, 96, 192, 64, 5),     # 300 blocks of 4 tokens -> 256 blocks of 4 or 5 (96-row chunks);
                                # the separate weight gradient's 300 blocks -> 256 as well
    # several rounds of blocks per CU, with fewer tokens per block than a
    # cos/sin group (one partial group per block)
    (4096, 64, 448, 64, 3),     # 1024 blocks of 4 tokens: four rounds
    (3840, 64, 448, 64, 5),     # 960 blocks of 4 tokens: the last round three quarters full
    (8192, 64, 192, 64, 1),     # 1024 blocks of 8 tokens, d = 256
    (2048, 128, 448, 64, 3),    # nh = 128: 512 blocks of 4 strided tokens
    (4096, 128, 192, 64, 7),    # nh = 128, d = 256: 512 blocks of 8 strided tokens
])
def test_fused_backward_matches_oracle_and_separate_calls(sq, nh, nope, pe, off):
    c = synthetic.case(sq, nh, nope, pe, seed=4000 + sq, pos_offset=off)
    print(f"\n[parity] fused bwd {c.name}", flush=True)
    dv = Dev(c)
    dO, dW = dv.bwd()
    dO, dW = gu.host_bits(dO), dW.cpu().numpy()
    gu.check_bf16(dO, oracle.bwd_dx(dv.dY, dv.W, dv.pos, c.theta, nope, pe), "fused dO")
    ref, mag = gu.dw_refs(dv.dY, dv.O, dv.pos, c.theta, nope, pe)
    gu.check_dw(dW, ref, "fused dW", mag)
    # dO is the same computation as postmix_bwd_dx, bit for bit
    np.testing.assert_array_equal(dO, gu.host_bits(dv.dx()))
    # dW: other token blocks, other order; each repeats bitwise
    dW_sep = dv.dw().cpu().numpy()
    gu.check_dw(dW_sep, ref, "separate dW", mag)
    for _ in range(3):
        dO2, dW2 = dv.bwd()
        np.testing.assert_array_equal(gu.host_bits(dO2), dO)
        np.testing.assert_array_equal(dW2.cpu().numpy(), dW)


def test_forward_only_workload_sq1024(kernel_policy):
    full_check(synthetic.CASES["fwd_1k"], ops=("fwd",))


def test_sweep_nh3_full():
    """[8192, 3, 448+64]: every element of Y, dO (separate and single-call)
    and dW (both) against the oracle."""
    full_check(synthetic.CASES["sweep_nh3"], ops=("fwd", "dx", "dw", "bwd"))


# --------------------------------------------------------------------------
# properties
# --------------------------------------------------------------------------

def test_identity_mix_keeps_nope_columns_bitwise():
    c = synthetic.case(37, 64, 448, 64, seed=321, pos_offset=16384)
    W = synthetic.f32_to_bf16_bits(np.eye(64, dtype=np.float32))
    dv = Dev(c, W=W, need_dy=False)
    Y = gu.host_bits(dv.fwd())
    np.testing.assert_array_equal(Y[..., :448], dv.O[..., :448])
    ref = oracle.fwd(dv.O, W, dv.pos, THETA, 448, 64)
    gu.check_bf16(Y, ref, "W=I Y")


# (sq, nh, nope, pe, split): ten shapes, from one head to 128, so every family
# of head-mix kernel is crossed: the fp32 small-head kernels (nh <= 4 on rows
# that are not a multiple of 128 channels), token-packed tiles with W staged
# block-diagonally (nh <= 32), exact and padded 32/64/96/128-row tiles, and
# the general kernel (nope + pe not a multiple of 128)
SPLIT_N_SHAPES = [
    (19, 1, 448, 64, 256),    # 32 tokens per tile (packed)
    (23, 3, 448, 64, 256),    # 21 tokens per 64-row tile, block-diagonal W
    (17, 4, 120, 16, 64),     # d = 136: the fp32 small-head kernel on both sides
    (21, 4, 448, 64, 128),    # 16 tokens per tile
    (13, 8, 448, 64, 384),    # 8 tokens per tile
    (11, 32, 448, 64, 256),   # exact 32-row tile
    (9, 20, 448, 64, 256),    # padded to 32 rows
    (7, 64, 448, 64, 256),    # the production tile
    (5, 96, 440, 64, 120),    # d = 504 and 120: the general kernel on both sides
    (5, 128, 448, 64, 384),   # 128 rows, heads split over wave groups
]


@pytest.mark.parametrize("sq,nh,nope,pe,split", SPLIT_N_SHAPES)
def test_channel_axis_splits_bitwise(sq, nh, nope, pe, split):
    """The channel axis is a pure N dimension (PR #1772 body item 1; the pages
    test their split-N GEMM for bitwise equality over ten shapes, small head
    counts among them): the first `split` (nope) channels of Y and of dO
    computed over the full width equal bit for bit the same channels computed
    on their own (split + 0 channels), and so do the separate and the
    single-call dO."""
    c = synthetic.case(sq, nh, nope, pe, seed=880 + nh, pos_offset=321)
    dv = Dev(c)
    Y, dO = gu.host_bits(dv.fwd()), gu.host_bits(dv.dx())
    s = synthetic.case(sq, nh, split, 0, seed=880 + nh, pos_offset=321)
    ds = Dev(s, O=np.ascontiguousarray(dv.O[..., :split]), W=dv.W,
             dY=np.ascontiguousarray(dv.dY[..., :split]), positions=dv.pos)
    np.testing.assert_array_equal(gu.host_bits(ds.fwd()), Y[..., :split])
    np.testing.assert_array_equal(gu.host_bits(ds.dx()), dO[..., :split])
    np.testing.assert_array_equal(gu.host_bits(dv.bwd()[0]), dO)


def test_zero_positions_equal_the_unrotated_mix_bitwise():
    c = synthetic.case(23, 64, 448, 64, seed=333)
    dv = Dev(c, positions=np.zeros(23, np.int32))
    Y = gu.host_bits(dv.fwd())
    flat = synthetic.case(23, 64, 512, 0, seed=333)
    dv2 = Dev(flat, O=dv.O, W=dv.W, dY=dv.dY)
    np.testing.assert_array_equal(Y, gu.host_bits(dv2.fwd()))
    np.testing.assert_array_equal(gu.host_bits(dv.dx()), gu.host_bits(dv2.dx()))


def test_out_of_range_positions_are_clamped_not_read_out_of_bounds():
    c = synthetic.case(6, 4, 48, 16, seed=55)
    pos = np.array([-5, 0, 3, 63, 64, 1000], np.int32)
    dv = Dev(c, positions=pos)
    cos, sin = P().postmix_rope_table(THETA, 16, 64)
    Y = P().postmix_fwd(dv.dO_, dv.dW_, cos, sin, dv.dpos, 48, 16)
    clamped = np.clip(pos, 0, 63)
    ref = oracle.fwd(dv.O, dv.W, clamped, THETA, 48, 16)
    gu.check_bf16(gu.host_bits(Y), ref, "clamped positions")


# nh = 64: general dx kernel and two separate calls; nh = 20 and 8: padded or
# token-packed tiles and the fused backward, reading W element-wise
@pytest.mark.parametrize("nh", [64, 20, 8])
def test_unaligned_W(nh):
    """W that is 2-byte but not 16-byte aligned: results on the oracle."""
    import torch
    c = synthetic.case(29, nh, 448, 64, seed=909, pos_offset=300)
    dv = Dev(c)
    store = torch.empty(nh * nh + 1, dtype=torch.bfloat16, device="cuda")
    Wv = store[1:].view(nh, nh)
    Wv.copy_(dv.dW_)
    assert Wv.data_ptr() % 16 == 2
    Y = P().postmix_fwd(dv.dO_, Wv, dv.cos, dv.sin, dv.dpos, c.nope, c.pe)
    gu.check_bf16(gu.host_bits(Y), oracle.fwd(dv.O, dv.W, dv.pos, c.theta, c.nope, c.pe), "Y, W+2")
    dO, dW = P().postmix_bwd(dv.ddY_, dv.dO_, Wv, dv.cos, dv.sin, dv.dpos, c.nope, c.pe)
    gu.check_bf16(gu.host_bits(dO), oracle.bwd_dx(dv.dY, dv.W, dv.pos, c.theta, c.nope, c.pe), "dO, W+2")
    dO_dx = P().postmix_bwd_dx(dv.ddY_, Wv, dv.cos, dv.sin, dv.dpos, c.nope, c.pe)
    np.testing.assert_array_equal(gu.host_bits(dO), gu.host_bits(dO_dx))
    ref, mag = gu.dw_refs(dv.dY, dv.O, dv.pos, c.theta, c.nope, c.pe)
    gu.check_dw(dW.cpu().numpy(), ref, "dW, W+2", mag)


def test_empty_token_range():
    import torch
    c = synthetic.case(0, 4, 48, 16, seed=1)
    O = torch.empty((0, 4, 64), dtype=torch.bfloat16, device="cuda")
    W = gu.dev_bf16(c.W())
    pos = torch.empty((0,), dtype=torch.int32, device="cuda")
    cos, sin = P().postmix_rope_table(THETA, 16, 8)
    assert P().postmix_fwd(O, W, cos, sin, pos, 48, 16).shape == (0, 4, 64)
    assert P().postmix_bwd_dx(O, W, cos, sin, pos, 48, 16).shape == (0, 4, 64)
    dW = torch.full((4, 4), float("nan"), device="cuda")
    P().postmix_bwd_dw(O, O, cos, sin, pos, 48, 16, out=dW)
    assert torch.equal(dW.cpu(), torch.zeros(4, 4))


@pytest.mark.parametrize("nh", [64, 3])   # MFMA tiles; fp32 vector kernel for small nh
def test_dw_repeatable_bitwise_small(nh):
    c = synthetic.case(300, nh, 448, 64, seed=444, pos_offset=100)
    dv = Dev(c)
    first = dv.dw().cpu().numpy()
    for _ in range(9):
        np.testing.assert_array_equal(dv.dw().cpu().numpy(), first)


def test_non_finite_input_spreads_only_within_its_packed_tile():
    """Non-finite inputs are outside the contract (the pages deal with finite
    training activations).  This pins down what happens: with nh <= 32 the
    tiled kernels pack several tokens into one MFMA contraction with W staged
    block-diagonally, so an Inf in one token turns the same output channel of
    the other tokens of its tile into NaN (0 * Inf).  Tokens of other tiles and
    other channels are untouched and match the oracle, and the general kernels
    keep every token apart."""
    c = synthetic.case(63, 3, 448, 64, seed=515, pos_offset=9)
    O = c.O().copy()
    O[5, 1, 10] = 0x7F80  # +Inf (bf16 bits)
    dv = Dev(c, O=O, need_dy=False)
    Y = gu.bf16_to_f64(gu.host_bits(dv.fwd()))
    bad = ~np.isfinite(Y)
    assert not bad[..., :10].any() and not bad[..., 11:].any(), "only channel 10 may be affected"
    toks = np.where(bad.any(axis=(1, 2)))[0]
    # token 5 and its tile-mates: one contiguous group of at most 64 // 3 tokens
    assert 5 in toks and toks.max() - toks.min() + 1 == len(toks) <= 64 // 3, toks
    print(f"\n[case] Inf in token 5: channel 10 non-finite for tokens {toks.min()}..{toks.max()}", flush=True)
    ref = oracle.fwd(O, dv.W, dv.pos, c.theta, c.nope, c.pe)
    keep = np.ones(Y.shape, bool)
    keep[toks, :, 10] = False
    gu.check_bf16(gu.host_bits(dv.fwd())[keep], ref[keep], "Y outside the Inf's tile column")
    prev = P().testing_set_general_kernels(True)
    try:
        Yg_bits = gu.host_bits(dv.fwd())
    finally:
        P().testing_set_general_kernels(prev)
    Yg = gu.bf16_to_f64(Yg_bits)
    assert set(np.where((~np.isfinite(Yg)).any(axis=(1, 2)))[0]) == {5}
    keep_g = np.ones(Y.shape, bool)
    keep_g[5, :, 10] = False
    gu.check_bf16(Yg_bits[keep_g], ref[keep_g], "Y (general kernels) outside token 5's column")
