"""Host-side route-ahead set measures on hand-made plans."""
import numpy as np

from sparse_moe_ffn_02_amd import route_ahead as ra


def test_union_of_skips_pads_and_masked_rows():
    ids = np.array([[3, 1, 7], [-1, -1, -1], [9, 3, 2]])
    assert ra.union_of(ids).tolist() == [1, 2, 3, 7, 9]
    assert ra.union_of(ids, np.array([1, 1, 0])).tolist() == [1, 3, 7]
    assert ra.union_of(np.zeros((0, 4), dtype=np.int32)).tolist() == []


def test_coverage_and_waste():
    assert ra.coverage([1, 2, 3, 4], [2, 4, 6]) == 2 / 3
    assert ra.waste([1, 2, 3, 4], [2, 4, 6]) == 2 / 4
    assert ra.coverage([], [5]) == 0.0 and ra.waste([], [5]) == 0.0
    assert ra.coverage([5], []) == 1.0 and ra.waste([5], []) == 1.0
    assert ra.coverage(range(256), [0, 255]) == 1.0
    assert ra.waste([7, 7, 8], [7]) == 0.5           # sets, not multisets


def test_row_agreement():
    planned = np.array([[1, 2, 3, 4], [5, 6, 7, 8], [0, 0, 0, 0]])
    used = np.array([[1, 2, 9, 10], [5, 6, 7, 8], [-1, -1, -1, -1]])
    assert ra.row_agreement(planned, used) == (0.5 + 1.0) / 2     # the all-pad row holds nothing
    assert ra.row_agreement(planned, used, np.array([0, 1, 1])) == 1.0
    assert ra.row_agreement(planned[:0], used[:0]) == 1.0
