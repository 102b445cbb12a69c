"""Slack-aware sparse augmentation on one GPU (oracle; test infrastructure only).

Source: FVAttn review page, section 1 (Key Terms, "Slack-Aware Sparse
Augmentation (SASA)"): after load balancing, ranks left with slack get
additional high-value sparse blocks; section 3 (Method & Key Results): the
SASA stage spends each rank's idle time after load balancing on extra
high-value blocks to improve quality.

The pages describe ranks that are GPUs and price work in blocks.  The
readings taken for one GPU, priced in what the attention kernel of this
implementation actually runs:

* a work item (G consecutive query blocks of one head) runs as one sequence
  of 64-key tiles: the union of its rows' selected key blocks, a key block
  holding key_block/64 tiles (the last block only the tiles its keys reach).
  An item costs its union tiles.
* ranks are the W workers of a longest-first assignment of the items in
  work-list order, made in batches (``schedule.lpt_batched``); the slack of
  worker w is s_w = M - L_w, with L_w its load and M = max_w L_w.
* a block that is already in its item's union costs nothing: every row of an
  item takes every block of the union that is eligible for it (j < valid_i).
  A block outside the union costs one key block of tiles (key_block/64,
  also for a ragged last block), and once paid for it is in the union, so
  every row of the item for which it is eligible takes it.
* worker w spends its slack on its last item (the one of the latest batch
  that reached it): extra tiles there leave every other choice of the
  batched assignment, and of a list schedule, unchanged (a worker that took
  no later item keeps taking none when its load grows), so no worker ends
  after M.  It buys floor(s_w / (key_block/64)) key blocks.
* the value of key block j for item g is the sum of its rows' routing
  probabilities P_ij over the rows for which j is eligible, added in member
  order from 0.0 (the pages name no other measure of a block's value).  With
  one price per block, taking the candidates in the order (value desc, j asc)
  maximises the value the budget buys.

``union_fill`` is the same with no slack: every row takes the eligible
blocks of its item's union, which leaves every union, and the kernel's work,
unchanged.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from .schedule import lpt_batched


def item_unions(mask, group: int) -> np.ndarray:
    """[B*H*ng, nbk] bool: the union of the selections of the G rows of every
    work item g = (b*H + h)*ng + i // G (the last item of a head may hold
    fewer rows)."""
    mask = np.asarray(mask) != 0
    B, H, nb, nbk = mask.shape
    ng = -(-nb // group)
    out = np.zeros((B * H, ng, nbk), dtype=bool)
    rows = mask.reshape(B * H, nb, nbk)
    for i in range(nb):
        out[:, i // group] |= rows[:, i]
    return out.reshape(B * H * ng, nbk)


def block_tiles(nbk: int, n_tokens: int, key_block: int) -> np.ndarray:
    """64-key tiles of every key block: key_block / 64, the last block the
    tiles its keys reach."""
    t = np.full(nbk, key_block // 64, dtype=np.int64)
    t[-1] = -(-(n_tokens - (nbk - 1) * key_block) // 64)
    return t


def block_value(p_rows, valid_rows, j: int) -> float:
    """Value of key block j for an item: P of the item's rows (in member
    order) for which j is eligible, added from 0.0."""
    v = 0.0
    for p, nv in zip(p_rows, valid_rows):
        if j < nv:
            v += float(p[j])
    return v


def buy_order(value, j: int):
    """Sort key of a candidate: value descending, then block ascending."""
    return (-value, j)


def budget_blocks(slack: int, per_block: int) -> int:
    """Key blocks a slack of `slack` tiles buys at per_block tiles each."""
    return slack // per_block


@dataclasses.dataclass
class Augmented:
    mask: np.ndarray        # [B,H,nb,nbk] uint8, the augmented selection
    row_cnt: np.ndarray     # [B,H,nb] int64
    row_idx: np.ndarray     # [B,H,nb,nbk] int32: ascending selection, then the remaining
                            # eligible blocks in the routing rank order, then -1
    head_cnt: np.ndarray    # [B,H] int64
    added: np.ndarray       # [B,H,nb] int64, blocks added per row
    worker_of: np.ndarray   # [items] int64, worker of each work item
    load: np.ndarray        # [W] int64, union tiles per worker before augmentation
    last_item: np.ndarray   # [W] int64, the item that takes the worker's slack (-1: none)
    slack: np.ndarray       # [W] int64, M - load
    paid: np.ndarray        # [W] int64, key blocks bought per worker
    paid_tiles: np.ndarray  # [W] int64, tiles they hold
    makespan: int
    union: np.ndarray       # [items, nbk] bool, every item's union after augmentation


def _fill(mask, unions, order, valid, group: int):
    """Row i of item g selects its own blocks and every block of unions[g]
    eligible for it; row_idx lists the selection ascending, then the row's
    other eligible blocks in the rank order `order`, then -1."""
    mask = np.asarray(mask).astype(np.uint8)
    B, H, nb, nbk = mask.shape
    ng = -(-nb // group)
    valid = np.full((B, H, nb), nbk, dtype=np.int64) if valid is None else np.asarray(valid, dtype=np.int64)
    order = np.asarray(order)
    new = mask.copy()
    uni = np.asarray(unions).reshape(B, H, ng, nbk)
    for i in range(nb):
        eligible = np.arange(nbk)[None, None, :] < valid[:, :, i, None]
        new[:, :, i] |= (uni[:, :, i // group] & eligible).astype(np.uint8)
    cnt = new.astype(np.int64).sum(-1)
    row_idx = np.full((B, H, nb, nbk), -1, dtype=np.int32)
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                sel = np.nonzero(new[b, h, i])[0]
                rest = [int(j) for j in order[b, h, i] if j < valid[b, h, i] and not new[b, h, i, j]]
                row_idx[b, h, i, :sel.size] = sel
                row_idx[b, h, i, sel.size:sel.size + len(rest)] = rest
    return new, cnt, row_idx


def augment(prob, mask, order, work_order, valid, group: int, num_workers: int, n_tokens: int,
            key_block: int) -> Augmented:
    """Slack-aware augmentation priced in union tiles.

    prob [B,H,nb,nbk] fp64 block probabilities; mask [B,H,nb,nbk] the
    selection; order [B,H,nb,nbk] each row's routing rank order (P desc, j
    asc); work_order the work list (item ids); valid [B,H,nb] (or None) the
    eligible blocks per row; group = query blocks per work item; num_workers
    = W; n_tokens and key_block give the tiles of each key block.
    """
    prob = np.asarray(prob, dtype=np.float64)
    mask = np.asarray(mask).astype(np.uint8)
    B, H, nb, nbk = mask.shape
    ng = -(-nb // group)
    valid = np.full((B, H, nb), nbk, dtype=np.int64) if valid is None else np.asarray(valid, dtype=np.int64)
    tiles = block_tiles(nbk, n_tokens, key_block)
    per_block = key_block // 64

    union = item_unions(mask, group)
    costs = (union * tiles[None, :]).sum(-1)
    worker_of, load, last_item = lpt_batched(costs, work_order, num_workers)
    makespan = int(load.max()) if load.size else 0
    slack = makespan - load

    new_union = union.copy()
    paid = np.zeros(num_workers, dtype=np.int64)
    paid_tiles = np.zeros(num_workers, dtype=np.int64)
    for w in range(num_workers):
        g = int(last_item[w])
        budget = budget_blocks(int(slack[w]), per_block)
        if g < 0 or budget == 0:
            continue
        bh, gi = divmod(g, ng)
        b, h = divmod(bh, H)
        members = list(range(gi * group, min(nb, (gi + 1) * group)))
        p_rows = [prob[b, h, i] for i in members]
        v_rows = [int(valid[b, h, i]) for i in members]
        nv = max(v_rows)
        cands = [j for j in range(nv) if not union[g, j]]
        value = {j: block_value(p_rows, v_rows, j) for j in cands}
        take = sorted(cands, key=lambda j: buy_order(value[j], j))[:budget]
        for j in take:
            new_union[g, j] = True
        paid[w] = len(take)
        paid_tiles[w] = int(sum(int(tiles[j]) for j in take))

    new_mask, cnt, row_idx = _fill(mask, new_union, order, valid, group)
    added = cnt - mask.astype(np.int64).sum(-1)
    return Augmented(new_mask, cnt, row_idx, cnt.sum(-1), added, worker_of, load, last_item,
                     slack.astype(np.int64), paid, paid_tiles, makespan, new_union)


@dataclasses.dataclass
class UnionFilled:
    mask: np.ndarray        # [B,H,nb,nbk] uint8
    row_cnt: np.ndarray     # [B,H,nb] int64
    row_idx: np.ndarray     # [B,H,nb,nbk] int32: ascending selection, then the remaining
                            # eligible blocks in the routing rank order, then -1
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
    new, cnt, row_idx = _fill(mask, item_unions(mask, group), order, valid, group)
    return UnionFilled(new, cnt, row_idx, cnt.sum(-1), cnt - mask.astype(np.int64).sum(-1))


def retained_mass(prob, mask) -> np.ndarray:
    """Sum of the block probabilities of the selected blocks, per row."""
    return (np.asarray(prob, dtype=np.float64) * (np.asarray(mask) != 0)).sum(-1)
