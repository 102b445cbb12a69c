"""Pins for the slack-aware augmentation oracle: a hand-worked example with
ties, brute force over candidate subsets (the added blocks carry the most
probability a worker's slack can buy), and invariants (makespan kept, every
row stays a prefix of its ranking, nothing added without slack or
candidates, causal eligibility)."""
import itertools
import math

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


def test_hand_example_two_workers():
    # costs [2, 1, 3, 1]; list 2, 0, 1, 3; LPT: 2->w0 (3), 0->w1 (2), 1->w1 (3),
    # 3->w0 (tie 3/3, lowest id) -> loads [4, 3], M = 4, slack [0, 1].
    # w1 holds rows 0 and 1; its best candidate is row 1, block 2 (P = 0.25).
    prob, mask, rc = _hand_case()
    a = oracle.augment(prob, mask, rc, None, 1, 0, 2)
    assert a.load.tolist() == [4, 3] and a.makespan == 4 and a.slack.tolist() == [0, 1]
    assert a.worker_of.tolist() == [1, 1, 0, 0]
    assert a.added[0, 0].tolist() == [0, 1, 0, 0]
    assert a.mask[0, 0, 1].tolist() == [0, 1, 1, 0]
    assert a.row_idx[0, 0, 1].tolist() == [1, 2, -1, -1]
    assert a.head_cnt[0, 0] == 8


def test_hand_example_three_workers_ties():
    # LPT: 2->w0 (3), 0->w1 (2), 1->w2 (1), 3->w2 (2): loads [3, 2, 2], slack [0, 1, 1].
    # w1 (row 0): blocks 2 and 3 tie at 0.125 -> the smaller index, 2.
    # w2 (rows 1, 3): row 1 block 2 and row 3 block 3 tie at 0.25 -> the smaller row, 1.
    prob, mask, rc = _hand_case()
    a = oracle.augment(prob, mask, rc, None, 1, 0, 3)
    assert a.slack.tolist() == [0, 1, 1]
    assert a.added[0, 0].tolist() == [1, 1, 0, 0]
    assert a.mask[0, 0, 0].tolist() == [1, 1, 1, 0]
    assert a.mask[0, 0, 1].tolist() == [0, 1, 1, 0]
    assert a.mask[0, 0, 3].tolist() == [0, 0, 1, 0]


def _routed(seed, B=1, H=2, N=300, d=8, block=64, p=0.6, causal=False):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, N, d)) * 2
    k = rng.standard_normal((B, H, N, d)) * 2
    return oracle.route(q, k, block, p, causal=causal)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("N,G,W", [(400, 1, 6), (320, 1, 4), (500, 2, 5)])
def test_brute_force_added_blocks_carry_max_mass(seed, N, G, W):
    r = _routed(seed, N=N, p=0.3 + 0.1 * seed)
    a = oracle.augment(r.prob, r.mask, r.row_cnt, r.valid, G, 0, W)
    nb = r.mask.shape[-1]
    ng = -(-nb // G)
    for w in range(W):
        rows = [(h, i) for h in range(2) for i in range(nb) if a.worker_of[h * ng + i // G] == w]
        cands = [(h, i, j) for (h, i) in rows for j in range(nb) if not r.mask[0, h, i, j]]
        kk = min(int(a.slack[w]), len(cands))
        added = [(h, i, j) for (h, i, j) in cands if a.mask[0, h, i, j]]
        assert len(added) == kk == a.added_per_worker[w]
        if kk == 0 or len(cands) > 16:
            continue
        best = max(math.fsum(r.prob[0, h, i, j] for (h, i, j) in sub)
                   for sub in itertools.combinations(cands, kk))
        got = math.fsum(r.prob[0, h, i, j] for (h, i, j) in added)
        assert got >= best * (1 - 1e-15)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("W", [1, 4, 16, 64])
def test_invariants(W, causal):
    r = _routed(10 + W, B=1, H=3, N=1000, block=64, p=0.7, causal=causal)
    G = 4
    a = oracle.augment(r.prob, r.mask, r.row_cnt, r.valid, G, 0, W)
    new_load = a.load + a.added_per_worker
    assert new_load.max() == a.makespan                       # the makespan is kept
    if W == 1:
        assert a.added.sum() == 0
    assert (a.mask >= r.mask).all() and (a.added >= 0).all()
    assert (a.row_cnt == r.row_cnt + a.added).all()
    assert (a.head_cnt == a.row_cnt.sum(-1)).all()
    # every row is still the first row_cnt blocks of its ranking
    ranked_sel = np.take_along_axis(a.mask, r.order, -1)
    want = (np.arange(a.mask.shape[-1]) < a.row_cnt[..., None]).astype(np.uint8)
    assert (ranked_sel == want).all()
    assert (oracle.retained_mass(r.prob, a.mask) >= oracle.retained_mass(r.prob, r.mask)).all()
    if causal:
        nb = a.mask.shape[-1]
        assert not (a.mask * np.triu(np.ones((nb, nb), dtype=np.uint8), 1)).any()
    # a worker with slack left over has no candidate left
    nb = a.mask.shape[-1]
    ng = -(-nb // G)
    left = a.slack - a.added_per_worker
    for w in np.nonzero(left > 0)[0]:
        items = np.nonzero(a.worker_of == w)[0]
        for g in items:
            bh, i0 = divmod(int(g), ng)
            rows = a.row_cnt.reshape(-1, nb)[bh, i0 * G:(i0 + 1) * G]
            vrows = r.valid.reshape(-1, nb)[bh, i0 * G:(i0 + 1) * G]
            assert (rows == vrows).all()


def test_nothing_to_add_at_p_one():
    r = _routed(3, p=1.0)
    a = oracle.augment(r.prob, r.mask, r.row_cnt, r.valid, 2, 0, 5)
    assert a.added.sum() == 0 and (a.mask == 1).all()


def test_windows_change_only_the_list():
    r = _routed(4, H=4, N=640, p=0.6)
    G = 2
    ng = -(-r.mask.shape[-1] // G)
    a1 = oracle.augment(r.prob, r.mask, r.row_cnt, r.valid, G, 0, 6)
    a2 = oracle.augment(r.prob, r.mask, r.row_cnt, r.valid, G, 2 * ng, 6)
    for a in (a1, a2):
        assert (a.load + a.added_per_worker).max() == a.makespan


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
