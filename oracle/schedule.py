"""Work ordering and load balance model (oracle; test infrastructure only).

Source: FVAttn review page, section 1 (Key Terms, "Runtime Load Balancing"):
after the sparse mask is fixed, the real per-head workload is profiled and
work is redistributed to shorten the critical path; section 2 (Motivation):
predicted or history-based layouts fail because workloads shift between
few-step inference steps; section 3 (Method & Key Results) reports the load
imbalance factor.  On one GPU the workers are compute units and the work
items are (batch, head, query-block) units whose cost is the number of
selected key blocks.

* work list: units sorted by cost descending, equal costs by unit id
  ascending (a stable sort), unit id = (b*H + h)*nb + i.  The list may be
  cut into windows of consecutive unit ids (whole heads): then it runs window
  by window, longest first inside each window.  The windows are not from the
  pages; they are this implementation's way of keeping the query blocks that
  run together on the K/V of a few heads.
* work items: the attention kernel of this implementation processes G
  consecutive query blocks of one head together (256 query rows: G = 4 for
  bf16 with 64-row blocks, 2 with 128-row blocks); for the work list an item
  costs the summed counts of its blocks, item id
  g = (b*H + h)*ceil(nb/G) + i//G.
* greedy longest-processing-time (LPT): in work-list order, each unit goes to
  the worker with the least load so far, ties to the lowest worker id.
  ``lpt_batched`` takes the list W positions at a time: the workers ranked
  by (load, id) before the batch take its items in that rank order (one
  each), so every choice of a batch can be made in parallel.
* "before": a contiguous static partition of the natural unit order, worker w
  taking units [floor(w*U/W), floor((w+1)*U/W)) -- the analogue of each rank
  owning a fixed group of whole heads.
* load imbalance factor (LIF) = max worker load / mean worker load (the page
  names the factor but prints no formula; max/mean is the reading taken).
"""
from __future__ import annotations

import heapq

import numpy as np


def group_costs(row_cnt, group: int) -> np.ndarray:
    """Cost of each work item: the sum of row_cnt over its G query blocks."""
    rc = np.asarray(row_cnt, dtype=np.int64)
    nb = rc.shape[-1]
    flat = rc.reshape(-1, nb)
    ng = -(-nb // group)
    pad = np.zeros((flat.shape[0], ng * group), dtype=np.int64)
    pad[:, :nb] = flat
    return pad.reshape(flat.shape[0], ng, group).sum(-1).reshape(-1)


def work_list(costs, window_units: int | None = None) -> np.ndarray:
    """Unit ids sorted by (window asc, cost desc, id asc); window = id // window_units
    (None or 0: a single window)."""
    costs = np.asarray(costs).reshape(-1)
    U = costs.size
    if not window_units or window_units >= U:
        return np.argsort(-costs, kind="stable").astype(np.int64)
    parts = []
    for lo in range(0, U, window_units):
        hi = min(U, lo + window_units)
        parts.append(lo + np.argsort(-costs[lo:hi], kind="stable"))
    return np.concatenate(parts).astype(np.int64)


def lpt_assign(costs, order, num_workers: int):
    """Greedy LPT over `order`; returns (worker_of [U], worker_load [W])."""
    costs = np.asarray(costs, dtype=np.int64).reshape(-1)
    heap = [(0, w) for w in range(num_workers)]
    heapq.heapify(heap)
    worker_of = np.empty(costs.size, dtype=np.int64)
    load = np.zeros(num_workers, dtype=np.int64)
    for u in order:
        l, w = heapq.heappop(heap)
        worker_of[u] = w
        load[w] = l + costs[u]
        heapq.heappush(heap, (int(load[w]), w))
    return worker_of, load


def lpt_batched(costs, order, num_workers: int):
    """Longest-first assignment in batches of num_workers list positions.

    Before each batch the workers are ranked by (load asc, id asc); the r-th
    item of the batch goes to the r-th ranked worker, so a batch gives every
    worker at most one item and all of a batch's choices can be made at once.
    Returns (worker_of [U], worker_load [W], last_item [W]): last_item[w] is
    the item of the latest batch that reached w (-1: none).
    """
    costs = np.asarray(costs, dtype=np.int64).reshape(-1)
    order = np.asarray(order, dtype=np.int64).reshape(-1)
    load = np.zeros(num_workers, dtype=np.int64)
    worker_of = np.full(costs.size, -1, dtype=np.int64)
    last_item = np.full(num_workers, -1, dtype=np.int64)
    for b in range(0, order.size, num_workers):
        ranked = sorted(range(num_workers), key=lambda w: (int(load[w]), w))
        for r, g in enumerate(order[b:b + num_workers]):
            w = ranked[r]
            worker_of[g] = w
            load[w] += costs[g]
            last_item[w] = g
    return worker_of, load, last_item


def static_partition_loads(costs, num_workers: int) -> np.ndarray:
    """Loads when worker w owns the contiguous natural-order slice of units."""
    costs = np.asarray(costs, dtype=np.int64).reshape(-1)
    U = costs.size
    load = np.zeros(num_workers, dtype=np.int64)
    for w in range(num_workers):
        lo, hi = (w * U) // num_workers, ((w + 1) * U) // num_workers
        load[w] = costs[lo:hi].sum()
    return load


def load_imbalance(loads) -> float:
    loads = np.asarray(loads, dtype=np.float64)
    mean = loads.mean()
    return float(loads.max() / mean) if mean > 0 else 1.0
