"""Pins for the scheduling model and the work accounting (no GPU)."""
import itertools

import numpy as np
import pytest

import oracle


def test_work_list_hand_example():
    costs = np.array([3, 5, 1, 5, 3, 2])
    # cost 5: units 1, 3; cost 3: units 0, 4; cost 2: unit 5; cost 1: unit 2
    assert oracle.work_list(costs).tolist() == [1, 3, 0, 4, 5, 2]


def test_work_list_windows_hand_example():
    costs = np.array([3, 5, 1, 5, 3, 2, 9, 0])
    # windows of 3 units: [3,5,1] -> 1,0,2 ; [5,3,2] -> 3,4,5 ; [9,0] -> 6,7
    assert oracle.work_list(costs, 3).tolist() == [1, 0, 2, 3, 4, 5, 6, 7]
    assert oracle.work_list(costs, 0).tolist() == oracle.work_list(costs).tolist()
    assert oracle.work_list(costs, 100).tolist() == oracle.work_list(costs).tolist()


def test_group_costs_hand_example():
    row_cnt = np.array([[[3, 5, 1, 4, 2], [1, 1, 1, 1, 9]]])       # B=1, H=2, nb=5
    assert oracle.group_costs(row_cnt, 2).tolist() == [8, 5, 2, 2, 2, 9]
    assert oracle.group_costs(row_cnt, 1).tolist() == row_cnt.reshape(-1).tolist()


def test_work_list_is_sorted_permutation():
    rng = np.random.default_rng(0)
    costs = rng.integers(0, 40, size=5000)
    wl = oracle.work_list(costs)
    assert sorted(wl.tolist()) == list(range(costs.size))
    c = costs[wl]
    assert (np.diff(c) <= 0).all()
    same = np.diff(c) == 0
    assert (np.diff(wl)[same] > 0).all()


def test_lpt_hand_example():
    costs = np.array([5, 4, 3, 3, 3])
    worker_of, load = oracle.lpt_assign(costs, oracle.work_list(costs), 2)
    assert worker_of.tolist() == [0, 1, 1, 0, 1]
    assert load.tolist() == [8, 10]
    assert oracle.load_imbalance(load) == pytest.approx(10 / 9)


def test_lpt_ties_go_to_lowest_worker():
    costs = np.array([1, 1, 1, 1])
    worker_of, load = oracle.lpt_assign(costs, oracle.work_list(costs), 3)
    assert worker_of.tolist() == [0, 1, 2, 0]


def _opt_makespan(costs, W):
    best = None
    for assign in itertools.product(range(W), repeat=len(costs)):
        loads = [0] * W
        for c, w in zip(costs, assign):
            loads[w] += c
        m = max(loads)
        best = m if best is None else min(best, m)
    return best


@pytest.mark.parametrize("seed", range(8))
def test_lpt_graham_bound_against_brute_force(seed):
    rng = np.random.default_rng(seed)
    W = 3
    costs = rng.integers(1, 20, size=int(rng.integers(4, 9)))
    _, load = oracle.lpt_assign(costs, oracle.work_list(costs), W)
    opt = _opt_makespan(costs.tolist(), W)
    assert load.max() <= (4 / 3 - 1 / (3 * W)) * opt + 1e-9
    assert load.max() <= costs.sum() / W + costs.max()
    assert load.sum() == costs.sum()


def test_static_partition_and_lif():
    costs = np.array([4, 4, 1, 1, 1, 1, 2, 2])
    load = oracle.static_partition_loads(costs, 4)
    assert load.tolist() == [8, 2, 2, 4]
    assert oracle.load_imbalance(load) == pytest.approx(8 / 4)
    assert oracle.load_imbalance([3, 3, 3]) == 1.0


def test_executed_flops_hand_and_dense():
    N, block, d = 130, 64, 8                                   # blocks of 64, 64, 2
    mask = np.zeros((1, 1, 3, 3), dtype=np.uint8)
    mask[0, 0, 0, [0, 2]] = 1
    mask[0, 0, 2, 1] = 1
    want = 4 * d * (64 * 64 + 64 * 2 + 2 * 64)
    assert oracle.executed_flops(mask, N, block, d) == want
    full = np.ones((2, 3, 3, 3), dtype=np.uint8)
    assert oracle.executed_flops(full, N, block, d) == oracle.dense_flops(2, 3, N, d)
    assert oracle.dense_flops(1, 1, 5, 2, causal=True) == 4 * 2 * 15
