"""Pins of the oracle planner (CPU only): the page's worked example, a
brute-force grouping written without any sort, and CSR invariants."""
import numpy as np
import pytest

import oracle


def brute_force_plan(slot_ids, S):
    """Group by scanning the slots in ascending order and appending token
    indices in ascending order: no sort, no library call."""
    order, indptr = [], [0]
    for s in range(S):
        for t, v in enumerate(slot_ids):
            if v == s:
                order.append(t)
        indptr.append(len(order))
    return order, indptr


def test_page_worked_example(golden):
    g = golden("plan_worked_example.txt")[""]
    S = int(g["S"][0])
    order, indptr, counts = oracle.plan(g["slot_ids"].astype(np.int32), S)
    np.testing.assert_array_equal(order, g["token_order"].astype(np.int32))
    np.testing.assert_array_equal(indptr, g["slot_indptr"].astype(np.int32))
    np.testing.assert_array_equal(counts, g["counts"].astype(np.int32))


@pytest.mark.parametrize("seed", range(20))
def test_against_brute_force(seed):
    g = np.random.default_rng(seed)
    S = int(g.integers(1, 40))
    T = int(g.integers(0, 300))
    slot_ids = g.integers(0, S, size=T).astype(np.int32)
    order, indptr, counts = oracle.plan(slot_ids, S)
    bo, bi = brute_force_plan(slot_ids.tolist(), S)
    assert order.tolist() == bo
    assert indptr.tolist() == bi
    # invariants: permutation, monotone offsets, histogram, stable
    assert sorted(order.tolist()) == list(range(T))
    assert indptr[0] == 0 and indptr[-1] == T and np.all(np.diff(indptr) >= 0)
    assert np.array_equal(np.diff(indptr), counts)
    for s in range(S):
        seg = order[indptr[s]:indptr[s + 1]]
        assert np.all(slot_ids[seg] == s) and np.all(np.diff(seg) > 0)


def test_rejects_bad_ids():
    with pytest.raises(ValueError):
        oracle.plan(np.array([0, 3], np.int32), 3)
    with pytest.raises(ValueError):
        oracle.plan(np.array([-1], np.int32), 3)


def test_work_list_covers_adapter_segments():
    slot_ids = np.array([3] * 40 + [0] * 5 + [1] * 3, np.int32)
    _, indptr, _ = oracle.plan(slot_ids, 5)
    wl = oracle.work_list(indptr, 16)
    assert wl.tolist() == [[1, 5, 3], [3, 8, 16], [3, 24, 16], [3, 40, 8]]
