"""Pins for the slack-aware augmentation oracle: a hand-worked example
(tests/golden/sasa_union_priced.json) with a batch that a sequential LPT
would assign differently, a tie and values that differ from one row's;
the batched LPT against the sequential one where they must agree; brute
force over candidate subsets (the bought blocks carry the most retained
mass the slack can buy); the assignment unchanged after augmentation with
the makespan kept; every row holding its item's union."""
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
    with open(os.path.join(golden_dir, "sasa_union_priced.json")) as f:
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
                              sh["n_tokens"], sh["key_block"])


def test_golden_union_priced_example(golden_dir):
    gd, a = _run_golden(golden_dir)
    ex = gd["expected"]
    assert a.worker_of.tolist() == ex["worker_of"]
    assert a.load.tolist() == ex["load"] and a.makespan == ex["makespan"]
    assert a.slack.tolist() == ex["slack"] and a.last_item.tolist() == ex["last_item"]
    assert a.paid.tolist() == ex["paid"] and a.paid_tiles.tolist() == ex["paid"]
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


# ------------------------------------------------- union-priced augmentation ---

def _routed(seed, B=1, H=2, N=300, d=8, block=64, p=0.6, causal=False, key_block=None):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, N, d)) * 2
    k = rng.standard_normal((B, H, N, d)) * 2
    return oracle.route(q, k, block, p, causal=causal, key_block=key_block)


def _augment(r, G, W, N, kb, window=0):
    order = oracle.work_list(oracle.group_costs(r.row_cnt, G), window)
    return oracle.augment(r.prob, r.mask, r.order, order, r.valid, G, W, N, kb)


def _mass_gain(prob, valid, rows, S):
    """Retained-mass gain of giving the blocks S to the rows (b, h, i), each
    where eligible, computed from masks."""
    gain = 0.0
    for (b, h, i) in rows:
        m = np.zeros(prob.shape[-1], dtype=bool)
        for j in S:
            if j < valid[b, h, i]:
                m[j] = True
        gain += float(oracle.retained_mass(prob[b, h, i], m))
    return gain


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("N,G,W,causal", [(400, 2, 5, False), (512, 4, 3, False), (640, 4, 4, True), (300, 1, 6, False)])
def test_brute_force_bought_blocks_carry_max_mass(seed, N, G, W, causal):
    r = _routed(seed, N=N, p=0.3 + 0.1 * seed, causal=causal)
    B, H, nb, nbk = r.mask.shape
    valid = r.valid if r.valid is not None else np.full((B, H, nb), nbk)
    a = _augment(r, G, W, N, 64)
    ng = -(-nb // G)
    old = oracle.item_unions(r.mask, G)
    for w in range(W):
        g = int(a.last_item[w])
        if g < 0:
            assert a.paid[w] == 0
            continue
        bh, gi = divmod(g, ng)
        b, h = divmod(bh, H)
        rows = [(b, h, i) for i in range(gi * G, min(nb, (gi + 1) * G))]
        nv = max(int(valid[x]) for x in rows)
        cands = [j for j in range(nv) if not old[g, j]]
        bought = [j for j in range(nbk) if a.union[g, j] and not old[g, j]]
        kk = min(int(a.slack[w]), len(cands))
        assert len(bought) == kk == a.paid[w]
        if kk == 0 or math.comb(len(cands), kk) > 5000:
            continue
        best = max(_mass_gain(r.prob, valid, rows, S) for S in itertools.combinations(cands, kk))
        assert _mass_gain(r.prob, valid, rows, bought) >= best * (1 - 1e-15)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("W,kb,N", [(1, 64, 1000), (4, 64, 1000), (16, 64, 1000), (64, 64, 1000),
                                    (8, 128, 1000), (24, 128, 1064)])
def test_assignment_unchanged_and_makespan_kept(W, kb, N, causal):
    # N = 1064 with 128-key blocks: a ragged last key block of one tile, so
    # some slacks are odd
    r = _routed(10 + W, B=1, H=3, N=N, block=64, p=0.3, causal=causal, key_block=kb)
    G = 4
    a = _augment(r, G, W, N, kb)
    tiles = oracle.block_tiles(r.mask.shape[-1], N, kb)
    new_costs = (a.union * tiles).sum(-1)
    old_costs = (oracle.item_unions(r.mask, G) * tiles).sum(-1)
    order = oracle.work_list(oracle.group_costs(r.row_cnt, G), 0)
    # priced in the tiles the kernel runs: the same assignment, every worker
    # grown by the tiles it bought, none past the makespan
    wo2, load2, last2 = oracle.lpt_batched(new_costs, order, W)
    assert wo2.tolist() == a.worker_of.tolist() and last2.tolist() == a.last_item.tolist()
    assert (load2 == a.load + a.paid_tiles).all() and load2.max() == a.makespan
    assert (a.paid * (kb // 64) >= a.paid_tiles).all()
    assert ((a.slack - a.paid * (kb // 64)) >= 0).all()
    # only last items grew
    grown = np.nonzero(new_costs != old_costs)[0]
    assert set(grown.tolist()) <= set(int(g) for g in a.last_item if g >= 0)
    if W == 1:
        assert a.paid.sum() == 0


@pytest.mark.parametrize("causal", [False, True])
def test_rows_take_their_item_union(causal):
    r = _routed(21, B=1, H=3, N=900, block=64, p=0.5, causal=causal)
    G = 4
    a = _augment(r, G, 7, 900, 64)
    B, H, nb, nbk = r.mask.shape
    ng = -(-nb // G)
    valid = r.valid if r.valid is not None else np.full((B, H, nb), nbk)
    for h in range(H):
        for i in range(nb):
            g = h * ng + i // G
            want = {j for j in np.nonzero(a.union[g])[0].tolist() if j < valid[0, h, i]}
            assert set(np.nonzero(a.mask[0, h, i])[0].tolist()) == want
            k = len(want)
            assert a.row_idx[0, h, i, :k].tolist() == sorted(want)
            ranked = [int(j) for j in r.order[0, h, i] if j < valid[0, h, i] and j not in want]
            assert a.row_idx[0, h, i, k:k + len(ranked)].tolist() == ranked
            assert (a.row_idx[0, h, i, k + len(ranked):] == -1).all()
    assert (a.mask >= r.mask).all()
    assert (a.row_cnt == r.mask.sum(-1) + a.added).all() and (a.head_cnt == a.row_cnt.sum(-1)).all()
    assert (oracle.retained_mass(r.prob, a.mask) >= oracle.retained_mass(r.prob, r.mask)).all()
    # a worker whose budget outlasted its candidates left its last item full
    for w in range(7):
        g = int(a.last_item[w])
        if g >= 0 and a.slack[w] > a.paid[w]:
            bh, gi = divmod(g, ng)
            nv = max(int(valid[0, bh, i]) for i in range(gi * G, min(nb, (gi + 1) * G)))
            assert a.union[g, :nv].all()


def test_nothing_to_buy_at_p_one():
    r = _routed(3, p=1.0)
    a = _augment(r, 2, 5, 300, 64)
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
