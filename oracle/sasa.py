"""Slack-aware sparse augmentation on one GPU (oracle; test infrastructure only).

Source: FVAttn review page, section 1 (Key Terms, "Slack-Aware Sparse
Augmentation (SASA)"): after load balancing, ranks left with slack get
additional high-value sparse blocks; section 3 (Method & Key Results): the
SASA stage spends each rank's idle time after load balancing on extra
high-value blocks to improve quality.

The pages describe ranks that are GPUs.  The reading taken for one GPU:

* ranks are the W workers of the longest-first LPT model (``schedule``):
  work items of G query blocks, item cost = summed selected-block counts,
  LPT over the head-windowed longest-first list;
* the slack of worker w is s_w = M - L_w, with L_w its LPT load and
  M = max_w L_w the modelled makespan, so augmenting keeps the makespan;
* the value of a key block j for query block i is its routing probability
  P_ij (the pages name no other measure of a block's value);
* the candidates of worker w are the eligible (j < valid_i: every block, or
  j <= i under causal routing) unselected key blocks of every query block of
  every item the LPT model gives to w;
* worker w adds the first min(s_w, #candidates) candidates in the order
  (P desc, unit asc, j asc).  Inside one row that is the routing rank order,
  so every row's selection stays a prefix of its ranking.  An added block
  costs one unit, like a selected one: L_w + added_w <= M.

A second reading works at the granularity of a work item instead of a
worker (``union_fill``): the attention kernel of this implementation runs a
work item of G query blocks as one sequence of key tiles, the union of the
G rows' selections, and a wave whose own row did not select a tile idles
through that step.  Those idle wave-steps are slack inside the item; filling
them costs no extra step.  So each row adds every eligible block of its
item's union that it did not select (all of them: they are free, so the
value order does not matter), which leaves every item's union, and with it
the kernel's work, unchanged.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from .schedule import group_costs, lpt_assign, work_list


@dataclasses.dataclass
class Augmented:
    mask: np.ndarray        # [B,H,nb,nb] uint8, the augmented selection
    row_cnt: np.ndarray     # [B,H,nb] int64
    row_idx: np.ndarray     # [B,H,nb,nb] int32, ascending selected indices, -1 after row_cnt
    head_cnt: np.ndarray    # [B,H] int64
    added: np.ndarray       # [B,H,nb] int64, blocks added per row
    worker_of: np.ndarray   # [items] int64, LPT worker of each work item
    load: np.ndarray        # [W] int64, LPT load before augmentation
    slack: np.ndarray       # [W] int64, M - load
    added_per_worker: np.ndarray   # [W] int64
    makespan: int


def augment(prob, mask, row_cnt, valid, group: int, window_items: int, num_workers: int) -> Augmented:
    """Slack-aware augmentation of a routed selection.

    prob [B,H,nb,nbk] fp64 block probabilities, mask [B,H,nb,nbk] the top-p
    selection, row_cnt [B,H,nb] its counts, valid [B,H,nb] (or None) the
    eligible blocks per row; group = query blocks per work item; window_items
    = items per scheduling window (0: one window); num_workers = W.
    """
    prob = np.asarray(prob, dtype=np.float64)
    mask = np.asarray(mask).astype(np.uint8)
    rc = np.asarray(row_cnt, dtype=np.int64)
    B, H, nb = rc.shape                       # nb query blocks per head
    nbk = mask.shape[-1]                      # key blocks per row
    valid = np.full((B, H, nb), nbk, dtype=np.int64) if valid is None else np.asarray(valid, dtype=np.int64)
    ng = -(-nb // group)

    costs = group_costs(rc, group)
    order = work_list(costs, window_items)
    worker_of, load = lpt_assign(costs, order, num_workers)
    makespan = int(load.max()) if load.size else 0
    slack = makespan - load

    # Every eligible unselected (unit, key block) pair with its worker and value.
    eligible = np.arange(nbk)[None, None, None, :] < valid[..., None]
    cand = eligible & (mask == 0)
    b_, h_, i_, j_ = np.nonzero(cand)
    unit = (b_ * H + h_) * nb + i_
    item = (b_ * H + h_) * ng + i_ // group
    wk = worker_of[item]
    p = prob[b_, h_, i_, j_]
    # Sorted by worker, then (P desc, unit asc, j asc); each worker keeps its first s_w.
    srt = np.lexsort((j_, unit, -p, wk))
    wk_s = wk[srt]
    start = np.searchsorted(wk_s, np.arange(num_workers), side="left")
    rank_in_worker = np.arange(srt.size) - start[wk_s]
    take = srt[rank_in_worker < slack[wk_s]]

    new_mask = mask.copy()
    new_mask[b_[take], h_[take], i_[take], j_[take]] = 1
    new_cnt = new_mask.astype(np.int64).sum(-1)
    row_idx = np.full((B, H, nb, nbk), -1, dtype=np.int32)
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                sel = np.nonzero(new_mask[b, h, i])[0]
                row_idx[b, h, i, :sel.size] = sel
    added_pw = np.bincount(wk[take], minlength=num_workers).astype(np.int64)
    return Augmented(new_mask, new_cnt, row_idx, new_cnt.sum(-1), new_cnt - rc, worker_of, load,
                     slack.astype(np.int64), added_pw, makespan)


@dataclasses.dataclass
class UnionFilled:
    mask: np.ndarray        # [B,H,nb,nbk] uint8
    row_cnt: np.ndarray     # [B,H,nb] int64
    row_idx: np.ndarray     # [B,H,nb,nbk] int32: ascending selection, then the remaining eligible
                            # blocks in the routing rank order, then -1
    head_cnt: np.ndarray    # [B,H] int64
    added: np.ndarray       # [B,H,nb] int64


def union_fill(mask, order, valid, group: int) -> UnionFilled:
    """Work-item slack filling: row i of item g = (i // group) selects every
    eligible block (j < valid_i) that any row of the item selected.

    mask [B,H,nb,nbk] the selection, order [B,H,nb,nbk] the routing rank
    order of each row (P desc, j asc), valid [B,H,nb] (or None: all) the
    eligible blocks per row.
    """
    mask = np.asarray(mask).astype(np.uint8)
    B, H, nb, nbk = mask.shape
    valid = np.full((B, H, nb), nbk, dtype=np.int64) if valid is None else np.asarray(valid, dtype=np.int64)
    new = mask.copy()
    for i0 in range(0, nb, group):
        members = range(i0, min(nb, i0 + group))
        union = np.zeros((B, H, nbk), dtype=bool)
        for i in members:
            union |= mask[:, :, i].astype(bool)
        for i in members:
            eligible = np.arange(nbk)[None, None, :] < valid[:, :, i, None]
            new[:, :, i] = (union & eligible).astype(np.uint8) | mask[:, :, i]
    cnt = new.astype(np.int64).sum(-1)
    row_idx = np.full((B, H, nb, nbk), -1, dtype=np.int32)
    order = np.asarray(order)
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                sel = np.nonzero(new[b, h, i])[0]
                rest = [int(j) for j in order[b, h, i] if j < valid[b, h, i] and not new[b, h, i, j]]
                row_idx[b, h, i, :sel.size] = sel
                row_idx[b, h, i, sel.size:sel.size + len(rest)] = rest
    return UnionFilled(new, cnt, row_idx, cnt.sum(-1), cnt - mask.astype(np.int64).sum(-1))


def retained_mass(prob, mask) -> np.ndarray:
    """Sum of the block probabilities of the selected blocks, per row."""
    return (np.asarray(prob, dtype=np.float64) * (np.asarray(mask) != 0)).sum(-1)
