"""The widest accepted rows: nope + pe = 2^24 channels per head, at the
largest head count (nh = 128), one token (4 GiB per tensor).

Offsets inside a token (head * d + channel) then reach 2^31 - 8, the end of
the 31-bit range the kernels index within a token.  d = 2^24 runs the tiled
forward and dx, the chunked dW and the fused backward; d = 2^24 - 8 (not a
multiple of 128) runs the general mix and the general dW.  Y and dO are
checked against the oracle at sampled elements (every head row's pe channels
among them), dW at sampled entries; the fused backward's dO is bitwise the
separate dx's, and its dW is checked the same way.

dW.  A partial's fp32 accumulation chain is capped at 2^14 MFMA k-steps
(16 channels each): the one token's 2^20 k-steps are split into 64 channel
spans, each with its own partial, which the fixed-order reduction adds.
Before the cap this case measured 1.05e-4 norm-wise (general kernel), above
the 1e-4 bar; the sampled entries are now held to the bar norm-wise and
each within 1e-4 of the largest sampled |entry|.
"""
import numpy as np
import pytest

import oracle
from tests import gpu_util as gu

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gu.has_gfx950(), reason="needs an MI355X (gfx950)")]

THETA = 10000.0


def P():
    from rope_head_mixing_amd import postmix
    return postmix


@pytest.mark.parametrize("nope,pe", [((1 << 24) - 64, 64), ((1 << 24) - 72, 64)])
def test_widest_rows_at_128_heads(nope, pe):
    import torch
    pm = P()
    sq, nh, d = 1, 128, nope + pe
    print(f"\n[case] wide rows sq={sq} nh={nh} nope={nope} pe={pe}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(d % 1000)
    O = torch.randn(sq, nh, d, device="cuda", generator=g).to(torch.bfloat16)
    dY = torch.randn(sq, nh, d, device="cuda", generator=g).to(torch.bfloat16)
    W = (torch.eye(nh, device="cuda") + 0.02 * torch.randn(nh, nh, device="cuda", generator=g)).to(torch.bfloat16)
    pos_h = np.array([12345], np.int32)
    pos = torch.from_numpy(pos_h).to("cuda")
    cos, sin = pm.postmix_rope_table(THETA, pe, 12346)
    ws = torch.empty(pm.postmix_bwd_dw_workspace_bytes(sq, nh, nope, pe), dtype=torch.uint8, device="cuda")

    Y = pm.postmix_fwd(O, W, cos, sin, pos, nope, pe)
    dO = pm.postmix_bwd_dx(dY, W, cos, sin, pos, nope, pe)
    dW = pm.postmix_bwd_dw(dY, O, cos, sin, pos, nope, pe, workspace=ws).cpu().numpy()
    dO_f, dW_f = pm.postmix_bwd(dY, O, W, cos, sin, pos, nope, pe, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(dO_f.view(torch.int16), dO.view(torch.int16))
    del dO_f
    dW_f = dW_f.cpu().numpy()

    rng = np.random.default_rng(11)
    chans = np.concatenate([np.arange(16), np.arange(d // 2 - 8, d // 2 + 8), np.arange(nope - 16, d)])
    heads = np.array([0, 1, 63, 64, 126, 127])
    idx = np.concatenate([(heads[:, None] * d + chans[None, :]).ravel(),
                          rng.integers(0, nh * d, 2048)]).astype(np.int64)
    idx_t = torch.from_numpy(idx).to("cuda")
    O_h, dY_h, W_h = gu.host_bits(O), gu.host_bits(dY), gu.host_bits(W)

    got = gu.host_bits(Y.reshape(-1)[idx_t])
    gu.check_bf16(got, oracle.fwd_at(O_h, W_h, pos_h, THETA, nope, pe, idx), "Y")
    got = gu.host_bits(dO.reshape(-1)[idx_t])
    gu.check_bf16(got, oracle.bwd_dx_at(dY_h, W_h, pos_h, THETA, nope, pe, idx), "dO")

    widx = np.concatenate([[0, nh * nh - 1, 127, 127 * nh], rng.integers(0, nh * nh, 28)])
    ref = oracle.bwd_dw_at(dY_h, O_h, pos_h, THETA, nope, pe, widx)
    for label, m in (("dW", dW), ("fused dW", dW_f)):
        got = m.reshape(-1)[widx].astype(np.float64)
        rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
        worst = float(np.abs(got - ref).max() / np.abs(ref).max())
        print(f"[case] {label}: sampled rel {rel:.3e}, max abs err / max abs {worst:.3e}", flush=True)
        assert rel <= gu.DW_REL, f"{label} sampled rel {rel:.3e}"
        assert worst <= gu.DW_REL, f"{label} max |err| / max |ref| {worst:.3e}"
