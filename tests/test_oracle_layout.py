"""Pins of the oracle's expert-contiguous layout: an independent stable sort
(numpy lexsort), closed-form invariants and the error cases."""
import numpy as np
import pytest

import oracle


def _case(S, T_src, k, E, local, seed):
    rng = np.random.default_rng(seed)
    topk = np.stack([rng.permutation(E)[:k] for _ in range(S * T_src)]).reshape(S, T_src, k)
    e2l = np.full(E, -1, np.int32)
    for i, e in enumerate(local):
        e2l[e] = i
    return topk.astype(np.int32), e2l


@pytest.mark.parametrize("S,T_src,k,E,local", [
    (1, 1, 1, 1, [0]),
    (1, 64, 2, 8, list(range(8))),
    (3, 65, 2, 8, [5, 1, 7]),          # remote experts, local order not id order
    (2, 1000, 6, 64, list(range(64))),
    (4, 37, 8, 256, [7, 39, 71, 103, 135, 167, 199, 231]),
])
def test_layout_equals_stable_sort(S, T_src, k, E, local):
    topk, e2l = _case(S, T_src, k, E, local, seed=S * 1000 + T_src)
    L = oracle.layout(topk, e2l, len(local))
    flat = topk.reshape(-1)
    le = e2l[flat]
    n = np.arange(flat.size)
    keep = le >= 0
    order = np.lexsort((n[keep], le[keep]))  # by local expert, then item index
    np.testing.assert_array_equal(L["row_src"], n[keep][order])
    np.testing.assert_array_equal(L["counts"], np.bincount(le[keep], minlength=len(local)))
    np.testing.assert_array_equal(L["offsets"], np.concatenate([[0], np.cumsum(L["counts"])]))
    assert L["R"] == keep.sum()
    # bijection: dest_row o row_src = identity, remote items -> -1
    np.testing.assert_array_equal(L["dest_row"][L["row_src"]], np.arange(L["R"]))
    assert np.all(L["dest_row"][~keep] == -1)
    if len(local) == E:
        assert L["R"] == S * T_src * k


def test_layout_empty_and_no_local():
    e2l = np.array([0, 1, -1, -1], np.int32)
    L = oracle.layout(np.zeros((2, 0, 2), np.int32), e2l, 2)
    assert L["R"] == 0 and list(L["offsets"]) == [0, 0, 0]
    topk, e2l = _case(1, 10, 2, 4, [], 1)
    L = oracle.layout(topk, np.full(4, -1, np.int32), 0)
    assert L["R"] == 0 and np.all(L["dest_row"] == -1)


def test_layout_errors():
    topk, e2l = _case(1, 10, 2, 4, [0, 1, 2, 3], 2)
    with pytest.raises(ValueError, match="R_cap"):
        oracle.layout(topk, e2l, 4, R_cap=19)
    bad = topk.copy()
    bad[0, 3, 1] = 4
    with pytest.raises(ValueError, match="out of range"):
        oracle.layout(bad, e2l, 4)
