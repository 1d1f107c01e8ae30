"""Pins for the oracle of the KV column index remap (PaddleFleet PR #1772, PR
body item 2 and description part 二: per-batch-local indices over a
[b*sq, topk] table become flat-global by adding b * seqlen_kv).

Pinned by a hand-worked table and by the composition the pages describe the
unfused route as (a fill, a >= 0 mask, a batch arange broadcast and scaled,
an add and a select), written with numpy primitives.
"""
import numpy as np
import pytest

import oracle


def test_hand_worked_table():
    # b = 2 batches of sq = 2 rows, topk = 3, seqlen_kv = 10, padding -1
    idx = np.array([[0, 4, -1],
                    [9, -1, -1],
                    [0, 3, 7],
                    [-1, 2, -5]], np.int32)
    want = np.array([[0, 4, -1],
                     [9, -1, -1],
                     [10, 13, 17],
                     [-1, 12, -1]], np.int32)
    np.testing.assert_array_equal(oracle.kv_remap(idx, sq=2, seqlen_kv=10), want)


def numpy_seven_steps(idx, sq, seqlen_kv, pad):
    """fill, greater_equal, arange, expand, scale, add, where."""
    rows, topk = idx.shape
    filled = np.full(idx.shape, pad, np.int64)
    valid = np.greater_equal(idx, 0)
    batch = np.arange(rows // sq, dtype=np.int64)
    batch = np.broadcast_to(np.repeat(batch, sq)[:, None], idx.shape)
    offset = batch * seqlen_kv
    shifted = idx.astype(np.int64) + offset
    return np.where(valid, shifted, filled).astype(np.int32)


@pytest.mark.parametrize("b,sq,topk,seqlen_kv,pad", [(3, 5, 7, 100, -1), (1, 16, 640, 65536, -1),
                                                     (4, 8, 2176, 1 << 20, -7), (2, 1, 1, 5, 0)])
def test_matches_the_seven_step_composition(b, sq, topk, seqlen_kv, pad):
    rng = np.random.default_rng(b * 1000 + topk)
    idx = rng.integers(-3, seqlen_kv, size=(b * sq, topk), dtype=np.int64).astype(np.int32)
    np.testing.assert_array_equal(oracle.kv_remap(idx, sq, seqlen_kv, pad),
                                  numpy_seven_steps(idx, sq, seqlen_kv, pad))


def test_rejects_rows_not_a_multiple_of_sq():
    with pytest.raises(ValueError):
        oracle.kv_remap(np.zeros((5, 3), np.int32), sq=2, seqlen_kv=10)
