"""Full-size parity: every element of every output at the production and
head-count-sweep workloads, against the fp64 oracle.

The workloads (rope_head_mixing_amd.synthetic.CASES):
  - prod: O and dY [16384, 64, 448+64] bf16 (1 GiB each), positions
    16384..32767 (one context-parallel shard of a 64K sequence, PaddleFleet
    PR #1772 body item 1), forward and backward;
  - sweep_nh128: [8192, 128, 448+64];
  - sweep_nh96 and sweep_nh72: [8192, 96 or 72, 448+64] (96-row tiles and
    chunks, 72 with padding rows);
  - a 20500-token production-width case whose single-call backward blocks
    hold 24 tokens (the staged cos/sin rows are refilled inside a block).
(The forward-only [1024, 64, 448+64] and the nh = 3 sweep are checked the
same way in test_parity_gpu.py.)

Each output is compared element by element: Y and dO (postmix_bwd_dx) with
the oracle computed 512 tokens at a time, dO of the single-call backward
(postmix_bwd) bit for bit against postmix_bwd_dx's, and every dW entry of both
backward entry points against the oracle's full weight gradient, with the
tolerances of tests/gpu_util.py.  Both dW results must also repeat bit for
bit over 10 runs, and so must the single-call dO.
"""
import numpy as np
import pytest

import oracle
from rope_head_mixing_amd import synthetic
from tests import gpu_util as gu
from tests.test_parity_gpu import Dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gu.has_gfx950(), reason="needs an MI355X (gfx950)")]


def P():
    from rope_head_mixing_amd import postmix
    return postmix


def full_size_check(case, repeat=10):
    import torch
    c = case
    print(f"\n[full] {c.name}: sq={c.sq} nh={c.nh} nope={c.nope} pe={c.pe} positions "
          f"{c.pos_offset}..{c.pos_offset + c.sq - 1}", flush=True)
    dv = Dev(c)
    res = {}

    Y = gu.host_bits(dv.fwd())
    res["Y"] = gu.check_bf16_streamed(
        Y, lambda s0, s1: oracle.fwd(dv.O[s0:s1], dv.W, dv.pos[s0:s1], c.theta, c.nope, c.pe), f"{c.name} Y")
    print(f"[full] {c.name}: Y every element, worst err/bound {res['Y']:.3f}", flush=True)
    del Y

    dO_t = dv.dx()
    dO = gu.host_bits(dO_t)
    res["dO"] = gu.check_bf16_streamed(
        dO, lambda s0, s1: oracle.bwd_dx(dv.dY[s0:s1], dv.W, dv.pos[s0:s1], c.theta, c.nope, c.pe),
        f"{c.name} dO")
    print(f"[full] {c.name}: dO every element, worst err/bound {res['dO']:.3f}", flush=True)
    del dO

    ws = torch.empty(P().postmix_bwd_dw_workspace_bytes(c.sq, c.nh, c.nope, c.pe), dtype=torch.uint8,
                     device="cuda")
    dO_f, dW_f = dv.bwd(workspace=ws)
    assert torch.equal(dO_f.view(torch.int16), dO_t.view(torch.int16)), "single-call dO != postmix_bwd_dx's"
    dW_f = dW_f.cpu().numpy()
    dW = dv.dw(workspace=ws).cpu().numpy()
    ref, mag = gu.dw_refs(dv.dY, dv.O, dv.pos, c.theta, c.nope, c.pe)
    res["dW"] = gu.check_dw(dW, ref, f"{c.name} dW", mag)
    res["fused dW"] = gu.check_dw(dW_f, ref, f"{c.name} fused dW", mag)
    print(f"[full] {c.name}: every dW entry, ||err||/||ref|| separate {res['dW']:.2e} "
          f"single-call {res['fused dW']:.2e}", flush=True)

    for _ in range(repeat - 1):
        np.testing.assert_array_equal(dv.dw(workspace=ws).cpu().numpy(), dW)
        dO_r, dW_r = dv.bwd(workspace=ws)
        np.testing.assert_array_equal(dW_r.cpu().numpy(), dW_f)
        assert torch.equal(dO_r.view(torch.int16), dO_t.view(torch.int16))
    print(f"[full] {c.name}: dW (both entry points) and dO bitwise identical over {repeat} runs", flush=True)
    return res


def test_production_forward_and_backward_every_element():
    """sq=16384, nh=64, 448+64, positions 16384..32767."""
    full_size_check(synthetic.CASES["prod"])


def test_sweep_nh128_every_element():
    """sq=8192, nh=128, 448+64, positions 0..8191."""
    full_size_check(synthetic.CASES["sweep_nh128"])


@pytest.mark.parametrize("name", ["sweep_nh96", "sweep_nh72"])
def test_sweep_96_row_kernels_every_element(name):
    """sq=8192, nh=96 and 72, 448+64: the 96-row forward/dx tiles and the
    96-row chunks of the single-call backward (rows 72..95 padding at 72)."""
    full_size_check(synthetic.CASES[name], repeat=3)


def test_fused_backward_long_blocks_every_element():
    """sq=20500, nh=64: the single-call backward's token blocks hold 24
    tokens (the last one 4), so its staged cos/sin rows are refilled after 16
    tokens inside every block."""
    full_size_check(synthetic.case(20500, 64, 448, 64, seed=6100, pos_offset=7), repeat=3)
