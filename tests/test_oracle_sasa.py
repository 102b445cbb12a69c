"""Pins for the slack-aware augmentation oracle: a hand-worked example
(tests/golden/sasa_slack_purchase.json) with a batch that a sequential LPT
would assign differently and a first candidate that does not fit; the
batched LPT against the sequential one where they must agree; the purchase
checked against item costs counted from the masks (the longest affordable
prefix of the value order); the assignment unchanged after augmentation with
the makespan kept; row lists and causal eligibility."""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle


def _hand_case():
    # One head, four query blocks, G = 1 (items are rows).
    prob = np.array([[0.5, 0.25, 0.125, 0.125],
                     [0.0625, 0.5, 0.25, 0.1875],
                     [0.25, 0.25, 0.25, 0.25],
                     [0.125, 0.125, 0.5, 0.25]])[None, None]
    mask = np.array([[1, 1, 0, 0],
                     [0, 1, 0, 0],
                     [1, 1, 1, 0],
                     [0, 0, 1, 0]], dtype=np.uint8)[None, None]
    return prob, mask, mask.sum(-1)


def _golden(golden_dir):
    with open(os.path.join(golden_dir, "sasa_slack_purchase.json")) as f:
        gd = json.load(f)
    sh = gd["shape"]
    prob = np.array(gd["prob_32nds"], dtype=np.float64)[None] / 32.0
    H, nb = sh["H"], sh["nb"]
    mask = np.zeros((1, H, nb, nb), dtype=np.uint8)
    for h in range(H):
        for i in range(nb):
            mask[0, h, i, gd["selected"][h][i]] = 1
    # rank order of every row: P descending, equal P by the smaller block
    order = np.array([[[sorted(range(nb), key=lambda j: (-prob[0, h, i, j], j)) for i in range(nb)]
                       for h in range(H)]])
    return gd, sh, prob, mask, order


def _run_golden(golden_dir):
    gd, sh, prob, mask, order = _golden(golden_dir)
    return gd, oracle.augment(prob, mask, order, gd["work_list"], None, sh["group"], sh["workers"],
                              sh["n_tokens"], sh["key_block"], sh["tile_fixed"])


def test_golden_slack_purchase_example(golden_dir):
    gd, a = _run_golden(golden_dir)
    ex = gd["expected"]
    assert a.worker_of.tolist() == ex["worker_of"]
    assert a.load.tolist() == ex["load"] and a.makespan == ex["makespan"]
    assert a.slack.tolist() == ex["slack"] and a.last_item.tolist() == ex["last_item"]
    assert a.paid.tolist() == ex["paid"] and a.paid_cost.tolist() == ex["paid_cost"]
    assert a.mask[0].tolist() == ex["mask"]
    assert a.row_cnt[0].tolist() == ex["row_cnt"]
    assert a.head_cnt[0].tolist() == ex["head_cnt"]
    assert a.row_idx[0].tolist() == ex["row_idx"]


# ------------------------------------------------------------ batched LPT ---

@pytest.mark.parametrize("seed", range(4))
def test_lpt_batched_single_batch_is_lpt(seed):
    # At most W items: one batch, the items in list order to the workers in id
    # order, which is what the sequential greedy does from all-zero loads.
    rng = np.random.default_rng(seed)
    W = int(rng.integers(3, 40))
    n = int(rng.integers(1, W + 1))
    costs = rng.integers(1, 50, size=n)
    order = rng.permutation(n)
    wb, lb, last = oracle.lpt_batched(costs, order, W)
    ws, ls = oracle.lpt_assign(costs, order, W)
    assert wb.tolist() == ws.tolist() and lb.tolist() == ls.tolist()
    assert wb[order].tolist() == list(range(n))
    assert last.tolist() == [int(order[w]) if w < n else -1 for w in range(W)]


@pytest.mark.parametrize("seed", range(4))
def test_lpt_batched_batches(seed):
    rng = np.random.default_rng(10 + seed)
    W = int(rng.integers(2, 12))
    n = int(rng.integers(W, 6 * W))
    costs = rng.integers(0, 30, size=n)
    order = rng.permutation(n)
    wo, load, last = oracle.lpt_batched(costs, order, W)
    assert (np.bincount(wo, weights=costs, minlength=W) == load).all()
    for b in range(0, n, W):
        batch = wo[order[b:b + W]]
        assert len(set(batch.tolist())) == batch.size          # one item per worker and batch
    for w in range(W):
        mine = [p for p in range(n) if wo[order[p]] == w]
        assert last[w] == (order[mine[-1]] if mine else -1)
    # equal costs: a round robin, loads within one item of each other
    wo2, l2, _ = oracle.lpt_batched(np.full(n, 7), order, W)
    assert l2.max() - l2.min() <= 7


# ---------------------------------------------------- slack purchase (SASA) ---

def _routed(seed, B=1, H=2, N=300, d=8, block=64, p=0.6, causal=False, key_block=None):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, N, d)) * 2
    k = rng.standard_normal((B, H, N, d)) * 2
    return oracle.route(q, k, block, p, causal=causal, key_block=key_block)


def _augment(r, G, W, N, kb, F, window=0):
    order = oracle.work_list(oracle.group_costs(r.row_cnt, G), window)
    return oracle.augment(r.prob, r.mask, r.order, order, r.valid, G, W, N, kb, F)


def _item_cost_from_masks(mask, g, G, N, kb, F):
    """The cost of item g counted from a mask: F * its union tiles plus the
    tiles of every row's selected blocks."""
    B, H, nb, nbk = mask.shape
    ng = -(-nb // G)
    bh, gi = divmod(g, ng)
    b, h = divmod(bh, H)
    rows = mask[b, h, gi * G:min(nb, (gi + 1) * G)].astype(bool)
    spb = kb // 64
    t = [spb] * (nbk - 1) + [-(-(N - (nbk - 1) * kb) // 64)]
    union = rows.any(0)
    return F * sum(t[j] for j in range(nbk) if union[j]) + sum(t[j] for r in rows for j in range(nbk) if r[j])


CASES = [(400, 2, 5, False, 64, 3), (512, 4, 3, False, 64, 3), (640, 4, 4, True, 64, 2),
         (300, 1, 6, False, 64, 3), (1064, 4, 7, False, 128, 3), (1064, 2, 5, True, 128, 1)]


@pytest.mark.parametrize("seed", range(5))
@pytest.mark.parametrize("N,G,W,causal,kb,F", CASES)
def test_purchase_is_the_longest_affordable_prefix(seed, N, G, W, causal, kb, F):
    # Counted from the masks, independently of the pair prices: the bought
    # pairs raise the item's cost by paid_cost <= slack, they are the first
    # pairs of the value order, and the next pair would not have fitted.
    r = _routed(seed, N=N, p=0.3 + 0.1 * seed, causal=causal, key_block=kb)
    B, H, nb, nbk = r.mask.shape
    valid = r.valid if r.valid is not None else np.full((B, H, nb), nbk)
    a = _augment(r, G, W, N, kb, F)
    ng = -(-nb // G)
    for w in range(W):
        g = int(a.last_item[w])
        if g < 0:
            assert a.paid[w] == 0
            continue
        bh, gi = divmod(g, ng)
        b, h = divmod(bh, H)
        rows = range(gi * G, min(nb, (gi + 1) * G))
        cands = sorted(((float(r.prob[b, h, i, j]), i, j) for i in rows for j in range(int(valid[b, h, i]))
                        if not r.mask[b, h, i, j]), key=lambda c: (-c[0], c[1], c[2]))
        bought = {(i, j) for i in rows for j in range(nbk) if a.mask[b, h, i, j] and not r.mask[b, h, i, j]}
        k = len(bought)
        assert k == a.paid[w] and bought == {(i, j) for _, i, j in cands[:k]}
        before = _item_cost_from_masks(r.mask, g, G, N, kb, F)
        assert _item_cost_from_masks(a.mask, g, G, N, kb, F) - before == a.paid_cost[w] <= a.slack[w]
        if k < len(cands):
            nxt = r.mask.copy()
            nxt[b, h, cands[k][1], cands[k][2]] = 1
            for _, i, j in cands[:k]:
                nxt[b, h, i, j] = 1
            assert _item_cost_from_masks(nxt, g, G, N, kb, F) - before > a.slack[w]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("W,kb,N,F", [(1, 64, 1000, 3), (4, 64, 1000, 3), (16, 64, 1000, 3), (64, 64, 1000, 2),
                                      (8, 128, 1000, 3), (24, 128, 1064, 3)])
def test_assignment_unchanged_and_makespan_kept(W, kb, N, F, causal):
    r = _routed(10 + W, B=1, H=3, N=N, block=64, p=0.3, causal=causal, key_block=kb)
    G = 4
    a = _augment(r, G, W, N, kb, F)
    old = oracle.item_costs(r.mask, G, N, kb, F)
    new = oracle.item_costs(a.mask, G, N, kb, F)
    order = oracle.work_list(oracle.group_costs(r.row_cnt, G), 0)
    # priced from the new masks: the same assignment, every worker grown by
    # what it bought, none past the makespan
    wo2, load2, last2 = oracle.lpt_batched(new, order, W)
    assert wo2.tolist() == a.worker_of.tolist() and last2.tolist() == a.last_item.tolist()
    assert (load2 == a.load + a.paid_cost).all() and load2.max() == a.makespan
    grown = np.nonzero(new != old)[0]
    assert set(grown.tolist()) <= set(int(g) for g in a.last_item if g >= 0)
    assert (a.mask >= r.mask).all() and (a.row_cnt == r.mask.sum(-1) + a.added).all()
    assert (a.head_cnt == a.row_cnt.sum(-1)).all()
    assert (oracle.retained_mass(r.prob, a.mask) >= oracle.retained_mass(r.prob, r.mask)).all()
    if W == 1:
        assert a.paid.sum() == 0


def test_row_lists_and_eligibility():
    r = _routed(21, B=1, H=3, N=900, block=64, p=0.3, causal=True)
    a = _augment(r, 4, 7, 900, 64, 3)
    assert a.paid.sum() > 0
    B, H, nb, nbk = r.mask.shape
    for h in range(H):
        for i in range(nb):
            sel = np.nonzero(a.mask[0, h, i])[0].tolist()
            assert all(j < r.valid[0, h, i] for j in sel)
            k = len(sel)
            assert a.row_idx[0, h, i, :k].tolist() == sel
            ranked = [int(j) for j in r.order[0, h, i] if j < r.valid[0, h, i] and j not in sel]
            assert a.row_idx[0, h, i, k:k + len(ranked)].tolist() == ranked
            assert (a.row_idx[0, h, i, k + len(ranked):] == -1).all()


def test_nothing_to_buy_at_p_one():
    r = _routed(3, p=1.0)
    a = _augment(r, 2, 5, 300, 64, 3)
    assert a.paid.sum() == 0 and a.added.sum() == 0 and (a.mask == 1).all()


# ------------------------------------------------ work-item slack (union fill) ---

def test_union_fill_hand_example():
    # G = 2: rows 0 and 1 form item 0, rows 2 and 3 item 1.
    prob, mask, rc = _hand_case()
    order = np.argsort(-prob, axis=-1, kind="stable")
    u = oracle.union_fill(mask, order, None, 2)
    assert u.mask[0, 0].tolist() == [[1, 1, 0, 0], [1, 1, 0, 0], [1, 1, 1, 0], [1, 1, 1, 0]]
    assert u.added[0, 0].tolist() == [0, 1, 0, 2]
    # row 3: selection {0, 1, 2} ascending, then its remaining block 3
    assert u.row_idx[0, 0, 3].tolist() == [0, 1, 2, 3]
    # row 1 (P = [.0625, .5, .25, .1875]): selection {0, 1}, then 2 and 3 by rank
    assert u.row_idx[0, 0, 1].tolist() == [0, 1, 2, 3]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("G", [1, 2, 4])
def test_union_fill_against_brute_force(G, causal):
    r = _routed(3 + G, H=3, N=700, block=64, p=0.6, causal=causal)
    u = oracle.union_fill(r.mask, r.order, r.valid, G)
    B, H, nb, nbk = r.mask.shape
    for h in range(H):
        for i in range(nb):
            g0 = (i // G) * G
            union = set()
            for m in range(g0, min(nb, g0 + G)):
                union |= set(np.nonzero(r.mask[0, h, m])[0].tolist())
            want = {j for j in union if j < r.valid[0, h, i]}
            assert set(np.nonzero(u.mask[0, h, i])[0].tolist()) == want
            k = len(want)
            assert u.row_idx[0, h, i, :k].tolist() == sorted(want)
            ranked = [int(j) for j in r.order[0, h, i] if j < r.valid[0, h, i] and j not in want]
            assert u.row_idx[0, h, i, k:k + len(ranked)].tolist() == ranked
            assert (u.row_idx[0, h, i, k + len(ranked):] == -1).all()
    assert (u.mask >= r.mask).all()
    # the union of every item, and so the attention kernel's tiles, is unchanged
    for i0 in range(0, nb, G):
        assert (u.mask[:, :, i0:i0 + G].any(2) == r.mask[:, :, i0:i0 + G].any(2)).all()
    assert (u.head_cnt == u.row_cnt.sum(-1)).all()
    assert (oracle.retained_mass(r.prob, u.mask) >= oracle.retained_mass(r.prob, r.mask)).all()
    if G == 1:
        assert u.added.sum() == 0
