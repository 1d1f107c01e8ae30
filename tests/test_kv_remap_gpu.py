"""KV column index remap on the GPU, bit-exact against the oracle.

Shapes follow the pages' tests of this fusion (PaddleFleet PR #1772, the
CI-stall commit): topk widths 640 and 2176 with sq trimmed to 1024, and a
one-row one-column launch first; plus batches > 1 so the offset is exercised,
a topk that is not a multiple of 4 (scalar path) and in-place use.
"""
import numpy as np
import pytest

import oracle
from tests import gpu_util as gu

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gu.has_gfx950(), reason="needs an MI355X (gfx950)")]


def P():
    from rope_head_mixing_amd import postmix
    return postmix


def table(b, sq, topk, seqlen_kv, seed, pad_frac=0.1):
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, seqlen_kv, size=(b * sq, topk), dtype=np.int64).astype(np.int32)
    pad = rng.random(idx.shape) < pad_frac
    idx[pad] = -1
    return idx


@pytest.mark.parametrize("b,sq,topk,seqlen_kv,pad_value", [
    (1, 1, 1, 7, -1),            # one row, one column
    (1, 1024, 640, 16384, -1),
    (1, 1024, 2176, 16384, -1),
    (3, 1024, 2176, 131072, -1),
    (4, 333, 640, 65536, 0),
    (3, 5, 7, 100, -9),          # topk % 4 != 0: scalar path
    (2, 64, 130, 1 << 20, -1),   # ragged topk, large offsets; a batch boundary inside a workgroup
    (6, 3, 8, 50, -1),           # batches shorter than a workgroup (vector path)
    (5, 2, 100, 1000, -3),
])
def test_kv_remap_matches_oracle_bitwise(b, sq, topk, seqlen_kv, pad_value):
    import torch
    idx = table(b, sq, topk, seqlen_kv, seed=b * 7 + topk)
    want = oracle.kv_remap(idx, sq, seqlen_kv, pad_value)
    got = P().postmix_kv_index_remap(torch.from_numpy(idx).cuda(), sq, seqlen_kv, pad_value)
    np.testing.assert_array_equal(got.cpu().numpy(), want)


def test_kv_remap_in_place():
    import torch
    idx = table(2, 512, 640, 4096, seed=5)
    want = oracle.kv_remap(idx, 512, 4096)
    t = torch.from_numpy(idx).cuda()
    P().postmix_kv_index_remap(t, 512, 4096, out=t)
    np.testing.assert_array_equal(t.cpu().numpy(), want)


def test_kv_remap_unaligned_view_takes_the_scalar_path():
    import torch
    idx = table(2, 16, 64, 1000, seed=6)
    store = torch.empty(idx.size + 1, dtype=torch.int32, device="cuda")
    view = store[1:].view(idx.shape)
    view.copy_(torch.from_numpy(idx))
    out = torch.empty(idx.size + 1, dtype=torch.int32, device="cuda")[1:].view(idx.shape)
    assert view.data_ptr() % 16 != 0
    P().postmix_kv_index_remap(view, 16, 1000, out=out)
    np.testing.assert_array_equal(out.cpu().numpy(), oracle.kv_remap(idx, 16, 1000))
