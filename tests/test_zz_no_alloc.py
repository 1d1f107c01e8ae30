"""The no-allocation backward, postmix_bwd_noalloc, through the C ABI.

It is postmix_bwd with the weight-gradient partials in the library's static
device scratch instead of a caller workspace, so its dO and dW must equal
postmix_bwd's bit for bit on the same inputs.  Two calls in a row, the
second with a smaller input (fewer partials than the first left in the
scratch), then a shape that takes the two separate computations.  The small
shapes are also checked against the fp64 oracle.
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


def _noalloc_vs_workspace(case, with_oracle):
    import torch
    print(f"\n[noalloc] {case.name}: partials "
          f"{P().postmix_bwd_dw_workspace_bytes(case.sq, case.nh, case.nope, case.pe)} bytes", flush=True)
    dv = Dev(case)
    dO_n, dW_n = P().postmix_bwd_noalloc(dv.ddY_, dv.dO_, dv.dW_, dv.cos, dv.sin, dv.dpos, case.nope, case.pe)
    dO_w, dW_w = dv.bwd()
    torch.cuda.synchronize()
    assert torch.equal(dO_n.view(torch.int16), dO_w.view(torch.int16)), "dO differs from postmix_bwd's"
    np.testing.assert_array_equal(dW_n.cpu().numpy(), dW_w.cpu().numpy())
    if with_oracle:
        gu.check_bf16(gu.host_bits(dO_n), oracle.bwd_dx(dv.dY, dv.W, dv.pos, case.theta, case.nope, case.pe),
                      f"{case.name} dO")
        ref, mag = gu.dw_refs(dv.dY, dv.O, dv.pos, case.theta, case.nope, case.pe)
        gu.check_dw(dW_n.cpu().numpy(), ref, f"{case.name} dW", mag)


def test_noalloc_backward_equals_postmix_bwd_on_consecutive_calls():
    # 4096 production-width tokens: 1024 partials of 64 x 64 (16 MiB of the scratch)
    _noalloc_vs_workspace(synthetic.case(4096, 64, 448, 64, seed=9100, pos_offset=16384), with_oracle=False)
    # then a smaller input: 8 heads, 300 tokens, packed chunks
    _noalloc_vs_workspace(synthetic.case(300, 8, 192, 64, seed=9200, pos_offset=5), with_oracle=True)
    # and a shape without the single pass (nh = 3 on rows that are not a
    # multiple of 128 channels): separate dx and dW, the dW partials again in the scratch
    _noalloc_vs_workspace(synthetic.case(77, 3, 120, 16, seed=9300, pos_offset=40), with_oracle=True)
