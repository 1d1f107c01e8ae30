"""Launches of more than 2^21 workgroups.

A data-sized launch of more than 2^21 workgroups takes rows of 2^21 in x and
the rows in y (one grid dimension holds fewer than 2^32 work-items).  These
cases are small shapes that reach a second row on their routes:

- the forward head mix in the token-part kernel at nh = 32, 64 + 64 channels
  (one tile per token): 2^21 + 4099 tokens, 17 GB per tensor;
- the small-head mix (nh <= 4, d not a multiple of 128) at one head of 16 pe
  channels, 256 tokens per workgroup: 2^29 + 5000 tokens, 17 GB;
- the full-width rotation (the unfused route's materialised inv_rope,
  PaddleFleet PR #1772, PR body item 1) at one head of 16 pe channels, where a
  workgroup covers one token;
- the KV index remap (PR body item 2) on its one-element-per-thread path
  (topk not a multiple of 4): 5.4e8 entries.

Y and the rotation are checked against the oracle on sampled tokens (both
grid rows and the seam between them), and bitwise against separate calls on
slices that fit one row.  The remap is checked against the oracle on every
entry.
"""
import numpy as np
import pytest

import oracle
from tests import gpu_util as gu

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gu.has_gfx950(), reason="needs an MI355X (gfx950)")]

ROW = 1 << 21  # workgroups per grid row


def P():
    from rope_head_mixing_amd import postmix
    return postmix


def _picks(sq, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([
        np.arange(64), np.arange(ROW - 64, ROW + 64), np.arange(sq - 4200, sq),
        rng.integers(0, sq, 2048)]))


def _sub(t, picks):
    import torch
    return t[torch.from_numpy(picks).to(t.device)].contiguous()


def test_forward_mix_over_two_grid_rows():
    import torch
    pm = P()
    sq, nh, nope, pe, theta = ROW + 4099, 32, 64, 64, 10000.0
    print(f"\n[case] postmix_fwd sq={sq} nh={nh} nope={nope} pe={pe}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(93)
    O = torch.randn(sq, nh, nope + pe, device="cuda", generator=g).to(torch.bfloat16)
    W = (torch.eye(nh, device="cuda") + 0.02 * torch.randn(nh, nh, device="cuda", generator=g)).to(torch.bfloat16)
    pos = (torch.arange(sq, device="cuda", dtype=torch.int64) * 3 % 65536).to(torch.int32)
    cos, sin = pm.postmix_rope_table(theta, pe, 65536)
    Y = pm.postmix_fwd(O, W, cos, sin, pos, nope, pe)
    torch.cuda.synchronize()

    picks = _picks(sq, 7)
    ref = oracle.fwd(gu.host_bits(_sub(O, picks)), gu.host_bits(W), _sub(pos, picks).cpu().numpy(),
                     theta, nope, pe)
    gu.check_bf16(gu.host_bits(_sub(Y, picks)), ref, "Y at sampled tokens")

    for lo, hi in [(0, 4096), (ROW - 2048, ROW + 2048), (sq - 4200, sq)]:
        part = pm.postmix_fwd(O[lo:hi].contiguous(), W, cos, sin, pos[lo:hi].contiguous(), nope, pe)
        np.testing.assert_array_equal(gu.host_bits(part), gu.host_bits(Y[lo:hi].contiguous()),
                                      err_msg=f"tokens [{lo}, {hi})")


def test_small_head_mix_over_two_grid_rows():
    import torch
    pm = P()
    tok = 256  # tokens per workgroup at 16 channels
    sq, nh, nope, pe, theta = ROW * tok + 5000, 1, 0, 16, 10000.0
    print(f"\n[case] postmix_fwd (small-head mix) sq={sq} nh={nh} nope={nope} pe={pe}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(95)
    O = torch.empty(sq, nh, nope + pe, device="cuda", dtype=torch.bfloat16)
    for lo in range(0, sq, 1 << 27):  # in slices: no full-size fp32 temporary
        hi = min(sq, lo + (1 << 27))
        O[lo:hi] = torch.randn(hi - lo, nh, nope + pe, device="cuda", generator=g).to(torch.bfloat16)
    W = torch.tensor([[1.25]], device="cuda").to(torch.bfloat16)
    pos = (torch.arange(sq, device="cuda", dtype=torch.int64) % 65536).to(torch.int32)
    cos, sin = pm.postmix_rope_table(theta, pe, 65536)
    Y = pm.postmix_fwd(O, W, cos, sin, pos, nope, pe)
    torch.cuda.synchronize()

    seam = ROW * tok
    rng = np.random.default_rng(9)
    picks = np.unique(np.concatenate([
        np.arange(64), np.arange(seam - 600, seam + 600), np.arange(sq - 5000, sq),
        rng.integers(0, sq, 2048)]))
    ref = oracle.fwd(gu.host_bits(_sub(O, picks)), gu.host_bits(W), _sub(pos, picks).cpu().numpy(),
                     theta, nope, pe)
    gu.check_bf16(gu.host_bits(_sub(Y, picks)), ref, "Y at sampled tokens")

    for lo, hi in [(0, 4096), (seam - 2048, seam + 2048), (sq - 5000, sq)]:
        part = pm.postmix_fwd(O[lo:hi].contiguous(), W, cos, sin, pos[lo:hi].contiguous(), nope, pe)
        np.testing.assert_array_equal(gu.host_bits(part), gu.host_bits(Y[lo:hi].contiguous()),
                                      err_msg=f"tokens [{lo}, {hi})")


def test_rotation_over_two_grid_rows():
    import torch
    pm = P()
    sq, nh, nope, pe, theta = ROW + 4099, 1, 0, 16, 10000.0
    print(f"\n[case] rope_apply sq={sq} nh={nh} nope={nope} pe={pe}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(91)
    X = torch.randn(sq, nh, nope + pe, device="cuda", generator=g).to(torch.bfloat16)
    pos = (torch.arange(sq, device="cuda", dtype=torch.int64) * 7 % 65536).to(torch.int32)
    cos, sin = pm.postmix_rope_table(theta, pe, 65536)
    out = pm.postmix_rope_apply(X, cos, sin, pos, nope, pe, -1)
    torch.cuda.synchronize()

    picks = _picks(sq, 5)
    got = gu.bf16_to_f64(gu.host_bits(_sub(out, picks)))
    ref = oracle.rotate(gu.bf16_to_f64(gu.host_bits(_sub(X, picks))), _sub(pos, picks).cpu().numpy(),
                        theta, nope, pe, -1)
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6)

    for lo, hi in [(0, 4096), (ROW - 2048, ROW + 2048), (sq - 4200, sq)]:
        part = pm.postmix_rope_apply(X[lo:hi].contiguous(), cos, sin, pos[lo:hi].contiguous(), nope, pe, -1)
        np.testing.assert_array_equal(gu.host_bits(part), gu.host_bits(out[lo:hi].contiguous()),
                                      err_msg=f"tokens [{lo}, {hi})")


def test_kv_remap_over_two_grid_rows():
    import torch
    pm = P()
    rows, sq, topk, seqlen_kv, pad = 257 * 1024, 1024, 2047, 2048, -5
    print(f"\n[case] kv_remap rows={rows} sq={sq} topk={topk} (one entry per thread)", flush=True)
    assert (rows * topk + 255) // 256 > ROW
    g = torch.Generator(device="cuda").manual_seed(17)
    idx = torch.randint(-1, seqlen_kv, (rows, topk), device="cuda", generator=g, dtype=torch.int32)
    out = pm.postmix_kv_index_remap(idx, sq, seqlen_kv, pad)
    torch.cuda.synchronize()
    ref = oracle.kv_remap(idx.cpu().numpy(), sq, seqlen_kv, pad)
    assert np.array_equal(out.cpu().numpy(), ref)
