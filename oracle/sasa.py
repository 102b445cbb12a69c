"""Slack-aware sparse augmentation on one GPU (oracle; test infrastructure only).

Source: FVAttn review page, section 1 (Key Terms, "Slack-Aware Sparse
Augmentation (SASA)"): after load balancing, ranks left with slack get
additional high-value sparse blocks; section 3 (Method & Key Results): the
SASA stage spends each rank's idle time after load balancing on extra
high-value blocks to improve quality.

The pages describe ranks that are GPUs and price work in blocks.  The
readings taken for one GPU, priced in what the attention kernel of this
implementation runs:

* a work item (G consecutive query blocks of one head) runs as one sequence
  of 64-key tiles, the union of its rows' selected key blocks (a key block
  holds key_block/64 tiles, the last block only the tiles its keys reach);
  every tile costs a fixed part and each row that selected it computes it.
  With row-tiles as the unit, an item costs
      F * (union tiles) + (row tiles),
  F = tile_fixed (a measured constant of the kernel, an input here).
* ranks are the W workers of a longest-first assignment of the items in
  work-list order, made in batches (``schedule.lpt_batched``); the slack of
  worker w is s_w = M - L_w, with L_w its cost and M = max_w L_w.
* worker w spends its slack on its last item (the one of the latest batch
  that reached it): extra cost there leaves every other choice of the
  batched assignment, and of a list schedule, unchanged (a worker that took
  no later item keeps taking none when its load grows), so no worker ends
  after M.
* its candidates are the (row, key block) pairs of that item whose block is
  eligible for the row and not selected by it; the value of a pair is the
  row's routing probability of the block (the pages name no other measure
  of a block's value).  Candidates go in the order (value desc, row asc,
  block asc); a pair costs the block's tiles t_j, plus F * t_j when its
  block is in neither the item's union nor an earlier pair of the order.
  The worker buys the longest prefix of that order whose total cost is at
  most s_w.

``union_fill`` gives every row of a work item the blocks of the item's
union that are eligible for it (the union, and the number of tiles, stay the
same; the row-tiles grow).
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


def buy_order(value, row: int, j: int):
    """Sort key of a candidate pair: value descending, then row, then block."""
    return (-value, row, j)


def pair_cost(tiles_j: int, opens: bool, tile_fixed: int) -> int:
    """Row-tiles of giving a row key block j: its tiles, plus the fixed part
    of every tile when the block is not yet in the item's union."""
    return tiles_j * (1 + (tile_fixed if opens else 0))


def item_costs(mask, group: int, n_tokens: int, key_block: int, tile_fixed: int) -> np.ndarray:
    """F * (union tiles) + (row tiles) of every work item."""
    mask = np.asarray(mask) != 0
    B, H, nb, nbk = mask.shape
    tiles = block_tiles(nbk, n_tokens, key_block)
    ng = -(-nb // group)
    row_tiles = (mask * tiles).sum(-1).reshape(B * H, nb)
    per_item = np.zeros((B * H, ng), dtype=np.int64)
    for i in range(nb):
        per_item[:, i // group] += row_tiles[:, i]
    union_tiles = (item_unions(mask, group) * tiles).sum(-1)
    return tile_fixed * union_tiles + per_item.reshape(-1)


@dataclasses.dataclass
class Augmented:
    mask: np.ndarray        # [B,H,nb,nbk] uint8, the augmented selection
    row_cnt: np.ndarray     # [B,H,nb] int64
    row_idx: np.ndarray     # [B,H,nb,nbk] int32: ascending selection, then the remaining
                            # eligible blocks in the routing rank order, then -1
    head_cnt: np.ndarray    # [B,H] int64
    added: np.ndarray       # [B,H,nb] int64, blocks added per row
    worker_of: np.ndarray   # [items] int64, worker of each work item
    load: np.ndarray        # [W] int64, cost per worker before augmentation
    last_item: np.ndarray   # [W] int64, the item that takes the worker's slack (-1: none)
    slack: np.ndarray       # [W] int64, M - load
    paid: np.ndarray        # [W] int64, pairs bought per worker
    paid_cost: np.ndarray   # [W] int64, their cost
    makespan: int


def _fill(mask, unions, order, valid, group: int):
    """Row i of item g selects its own blocks and every block of unions[g]
    eligible for it; row_idx as in _rebuild."""
    mask = np.asarray(mask).astype(np.uint8)
    B, H, nb, nbk = mask.shape
    valid = np.full((B, H, nb), nbk, dtype=np.int64) if valid is None else np.asarray(valid, dtype=np.int64)
    ng = -(-nb // group)
    new = mask.copy()
    uni = np.asarray(unions).reshape(B, H, ng, nbk)
    for i in range(nb):
        eligible = np.arange(nbk)[None, None, :] < valid[:, :, i, None]
        new[:, :, i] |= (uni[:, :, i // group] & eligible).astype(np.uint8)
    cnt = new.astype(np.int64).sum(-1)
    return new, cnt, _rebuild(new, np.asarray(order), valid)


def _rebuild(new, order, valid):
    """row_idx of a selection: ascending selected blocks, then the row's other
    eligible blocks in the rank order `order`, then -1."""
    B, H, nb, nbk = new.shape
    row_idx = np.full((B, H, nb, nbk), -1, dtype=np.int32)
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                sel = np.nonzero(new[b, h, i])[0]
                rest = [int(j) for j in order[b, h, i] if j < valid[b, h, i] and not new[b, h, i, j]]
                row_idx[b, h, i, :sel.size] = sel
                row_idx[b, h, i, sel.size:sel.size + len(rest)] = rest
    return row_idx


def augment(prob, mask, order, work_order, valid, group: int, num_workers: int, n_tokens: int,
            key_block: int, tile_fixed: int) -> Augmented:
    """Slack-aware augmentation priced in row-tiles.

    prob [B,H,nb,nbk] fp64 block probabilities; mask [B,H,nb,nbk] the
    selection; order [B,H,nb,nbk] each row's routing rank order (P desc, j
    asc); work_order the work list (item ids); valid [B,H,nb] (or None) the
    eligible blocks per row; group = query blocks per work item; num_workers
    = W; n_tokens and key_block give the tiles of each key block; tile_fixed
    = F, the fixed cost of a tile in row-tiles.
    """
    prob = np.asarray(prob, dtype=np.float64)
    mask = np.asarray(mask).astype(np.uint8)
    B, H, nb, nbk = mask.shape
    ng = -(-nb // group)
    valid = np.full((B, H, nb), nbk, dtype=np.int64) if valid is None else np.asarray(valid, dtype=np.int64)
    tiles = block_tiles(nbk, n_tokens, key_block)

    union = item_unions(mask, group)
    costs = item_costs(mask, group, n_tokens, key_block, tile_fixed)
    worker_of, load, last_item = lpt_batched(costs, work_order, num_workers)
    makespan = int(load.max()) if load.size else 0
    slack = makespan - load

    new = mask.copy()
    paid = np.zeros(num_workers, dtype=np.int64)
    paid_cost = np.zeros(num_workers, dtype=np.int64)
    for w in range(num_workers):
        g = int(last_item[w])
        if g < 0 or slack[w] <= 0:
            continue
        bh, gi = divmod(g, ng)
        b, h = divmod(bh, H)
        cands = [(i, j) for i in range(gi * group, min(nb, (gi + 1) * group))
                 for j in range(int(valid[b, h, i])) if not mask[b, h, i, j]]
        cands.sort(key=lambda c: buy_order(float(prob[b, h, c[0], c[1]]), c[0], c[1]))
        opened = union[g].copy()
        spent = 0
        for i, j in cands:
            c = pair_cost(int(tiles[j]), not opened[j], tile_fixed)
            if spent + c > slack[w]:
                break
            spent += c
            opened[j] = True
            new[b, h, i, j] = 1
            paid[w] += 1
        paid_cost[w] = spent

    cnt = new.astype(np.int64).sum(-1)
    row_idx = _rebuild(new, order, valid)
    added = cnt - mask.astype(np.int64).sum(-1)
    return Augmented(new, cnt, row_idx, cnt.sum(-1), added, worker_of, load, last_item,
                     slack.astype(np.int64), paid, paid_cost, makespan)


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
