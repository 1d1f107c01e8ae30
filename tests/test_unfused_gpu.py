"""The unfused comparison route on the GPU (PaddleFleet PR #1772, PR body
item 1: the unfused path materialises inv_rope(O) before the postmix GEMM;
the follow-up commit's final backward rebuilds it and runs the GEMM's
gradients, then the RoPE backward).

postmix_rope_apply is checked against the oracle's rotation; the unfused
forward and backward, composed of library entry points only, are checked
against the oracle at the same tolerance as the fused path (the extra bf16
rounding of the materialised tensor stays far inside it).
"""
import numpy as np
import pytest

import oracle
from rope_head_mixing_amd import synthetic
from tests import gpu_util as gu

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gu.has_gfx950(), reason="needs an MI355X (gfx950)")]


def P():
    from rope_head_mixing_amd import postmix
    return postmix


@pytest.mark.parametrize("sq,nh,nope,pe,off", [
    (37, 64, 448, 64, 16384),   # the production row shape, 4 head rows per workgroup
    (9, 4, 48, 16, 3),
    (5, 3, 0, 32, 1000),        # no nope channels; fewer heads than rows per workgroup
    (4, 7, 464, 16, 11),        # 60 vectors per row: 16 idle threads, a ragged head group
    (3, 5, 2048, 64, 7),        # 264 vectors per row: one row per workgroup, looped
])
@pytest.mark.parametrize("direction", [-1, +1])
def test_rope_apply_matches_oracle_rotation(sq, nh, nope, pe, off, direction):
    c = synthetic.case(sq, nh, nope, pe, seed=60 + sq, pos_offset=off)
    O, pos = c.O(), c.positions()
    cos, sin = P().postmix_rope_table(c.theta, pe, int(pos.max()) + 1)
    out = P().postmix_rope_apply(gu.dev_bf16(O), cos, sin, gu.dev_i32(pos), nope, pe, direction)
    got = gu.bf16_to_f64(gu.host_bits(out))
    ref = oracle.rotate(gu.bf16_to_f64(O), pos, c.theta, nope, pe, direction)
    # one bf16 rounding of the fp32 result: within 2^-8 relative (plus fp32 table error)
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6)
    np.testing.assert_array_equal(gu.host_bits(out)[..., :nope], O[..., :nope])


def check_with_intermediate_rounding(gpu_bits, ref, extra, label):
    """|gpu - ref| <= 1e-2 |ref| + 1e-3 + extra, where `extra` bounds the one
    additional bf16 rounding the unfused route makes of its materialised
    intermediate (derived per element below)."""
    got = gu.bf16_to_f64(gpu_bits)
    bound = gu.Y_RTOL * np.abs(ref) + gu.Y_ATOL + extra
    bad = np.abs(got - ref) > bound
    assert not bad.any(), f"{label}: {int(bad.sum())} elements beyond the derived bound"


@pytest.mark.parametrize("sq,nh,nope,pe,off", [(67, 64, 448, 64, 16384), (33, 20, 40, 16, 5)])
def test_unfused_route_matches_oracle(sq, nh, nope, pe, off):
    """The unfused route rounds X = inv_rope(O) (forward) and dX = W^T dY
    (backward) to bf16 before the next step.  A bf16 rounding moves a value by
    at most 2^-9 of itself, so the forward output moves by at most
    2^-9 sum_h |W[g,h]| |X[h,c]|, and the rotated dO by at most 2^-9 (|dX|_c +
    |dX|_partner) with |dX| <= |W|^T |dY|; 2^-8 is used for margin.  The fused
    path has no such term."""
    c = synthetic.case(sq, nh, nope, pe, seed=80 + sq, pos_offset=off)
    O, W, dY, pos = c.O(), c.W(), c.dY(), c.positions()
    cos, sin = P().postmix_rope_table(c.theta, pe, int(pos.max()) + 1)
    args = (cos, sin, gu.dev_i32(pos), nope, pe)
    Wf, Of, dYf = (gu.bf16_to_f64(x) for x in (W, O, dY))
    X = oracle.inv_rope(Of, pos, c.theta, nope, pe)

    Y = P().unfused_fwd(gu.dev_bf16(O), gu.dev_bf16(W), *args)
    extra_y = 2.0 ** -8 * np.einsum("gh,shc->sgc", np.abs(Wf), np.abs(X))
    check_with_intermediate_rounding(gu.host_bits(Y), oracle.fwd(O, W, pos, c.theta, nope, pe),
                                     extra_y, "unfused Y")

    dO, dW = P().unfused_bwd(gu.dev_bf16(dY), gu.dev_bf16(O), gu.dev_bf16(W), *args)
    a = np.einsum("gh,sgc->shc", np.abs(Wf), np.abs(dYf))
    h2 = pe // 2
    pair = a.copy()
    pair[..., nope:nope + h2] += a[..., nope + h2:]
    pair[..., nope + h2:] += a[..., nope:nope + h2]
    check_with_intermediate_rounding(gu.host_bits(dO), oracle.bwd_dx(dY, W, pos, c.theta, nope, pe),
                                     2.0 ** -8 * pair, "unfused dO")
    # dW of the unfused route multiplies dY by the bf16-rounded X: each term
    # moves by at most 2^-9 |dY||X| (one operand rounding; the fused path splits
    # that operand into hi + lo instead and meets 1e-4), plus fp32 summation
    ref_dw = oracle.bwd_dw(dY, O, pos, c.theta, nope, pe)
    bound = 2.0 ** -8 * np.einsum("sgc,shc->gh", np.abs(dYf), np.abs(X)) + 1e-5 * np.abs(ref_dw).max()
    assert np.all(np.abs(dW.cpu().numpy() - ref_dw) <= bound), "unfused dW beyond the derived bound"
