"""Pins for the routing oracle: hand-worked fixtures, brute force over subsets,
closed forms and invariants (no GPU)."""
import itertools
import json
import math
import os
import re

import numpy as np
import pytest
import scipy.special

import oracle


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- pooling ---

def test_pool_and_scores_hand_example(golden_dir):
    g = _load(golden_dir, "pool_scores_example.json")
    q = np.array(g["q"], dtype=np.float64)[None, None]
    k = np.array(g["k"], dtype=np.float64)[None, None]
    qbar = oracle.pool_blocks(q, g["block"])
    kbar = oracle.pool_blocks(k, g["block"])
    np.testing.assert_array_equal(qbar[0, 0], np.array(g["qbar"], dtype=np.float64))
    np.testing.assert_array_equal(kbar[0, 0], np.array(g["kbar"], dtype=np.float64))
    z = oracle.block_scores(qbar, kbar, g["scale"])
    np.testing.assert_array_equal(z[0, 0], np.array(g["scores"], dtype=np.float64))


def test_pool_constant_blocks_with_ragged_tail():
    rng = np.random.default_rng(0)
    B, H, N, d, block = 2, 3, 77, 5, 16           # 5 blocks, the last holds 13 tokens
    nb = oracle.num_blocks(N, block)
    assert nb == 5 and list(oracle.block_sizes(N, block)) == [16, 16, 16, 16, 13]
    const = rng.integers(-8, 8, size=(B, H, nb, d)).astype(np.float64)
    x = np.repeat(const, block, axis=2)[:, :, :N]
    np.testing.assert_array_equal(oracle.pool_blocks(x, block), const)


def test_pool_matches_token_loop():
    rng = np.random.default_rng(1)
    B, H, N, d, block = 1, 2, 37, 3, 8
    x = rng.standard_normal((B, H, N, d))
    got = oracle.pool_blocks(x, block)
    for b in range(B):
        for h in range(H):
            for i in range(oracle.num_blocks(N, block)):
                toks = [t for t in range(N) if t // block == i]
                for c in range(d):
                    want = math.fsum(x[b, h, t, c] for t in toks) / len(toks)
                    assert abs(got[b, h, i, c] - want) <= 1e-15 * (1 + abs(want))


# ---------------------------------------------------------------- softmax ---

def test_softmax_rows_library_and_sum():
    rng = np.random.default_rng(2)
    z = rng.standard_normal((3, 4, 17)) * 20
    p = oracle.softmax_rows(z)
    np.testing.assert_allclose(p, scipy.special.softmax(z, axis=-1), rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=0, atol=1e-14)
    assert (p >= 0).all()


# ------------------------------------------------------------------ top-p ---

def test_topp_golden_rows(golden_dir):
    g = _load(golden_dir, "topp_rows.json")
    for case in g["cases"]:
        prob = np.array(case["prob"], dtype=np.float64)[None, None, None]
        order, cum, cnt = oracle.top_p_select(prob, case["top_p"])
        assert list(order[0, 0, 0]) == case["ranked"], case
        assert list(cum[0, 0, 0]) == case["cum"], case
        assert int(cnt[0, 0, 0]) == case["count"], case
        assert sorted(order[0, 0, 0, : case["count"]].tolist()) == case["selected"], case


def _brute_force_topp(prob_row, p):
    """Smallest subset whose mass reaches p; among those, the largest mass."""
    nb = len(prob_row)
    if p >= 1:
        return set(range(nb))
    for size in range(1, nb + 1):
        best, best_mass = None, -1.0
        for sub in itertools.combinations(range(nb), size):
            mass = math.fsum(prob_row[j] for j in sub)
            if mass >= p and mass > best_mass:
                best, best_mass = set(sub), mass
        if best is not None:
            return best
    return set(range(nb))


@pytest.mark.parametrize("nb", [1, 2, 3, 4, 7, 10])
@pytest.mark.parametrize("p", [0.05, 0.3, 0.5, 0.75, 0.9, 0.99])
def test_topp_brute_force_subsets(nb, p):
    rng = np.random.default_rng(100 * nb + int(p * 100))
    for trial in range(6):
        z = rng.standard_normal(nb) * rng.uniform(0.1, 4)
        prob = scipy.special.softmax(z)
        order, cum, cnt = oracle.top_p_select(prob[None, None, None], p)
        got = set(order[0, 0, 0, : cnt[0, 0, 0]].tolist())
        assert got == _brute_force_topp(prob, p), (nb, p, prob)


def test_topp_invariants_prefix_reaches_p_minimally():
    rng = np.random.default_rng(3)
    prob = scipy.special.softmax(rng.standard_normal((2, 3, 20, 20)) * 3, axis=-1)
    for p in (0.1, 0.5, 0.9, 0.95):
        order, cum, cnt = oracle.top_p_select(prob, p)
        ranked = np.take_along_axis(prob, order, -1)
        assert (np.diff(ranked, axis=-1) <= 0).all()          # descending
        k = cnt[..., None]
        c_k = np.take_along_axis(cum, k - 1, -1)
        c_km1 = np.where(k >= 2, np.take_along_axis(cum, np.maximum(k - 2, 0), -1), 0.0)
        assert (c_k >= p).all() and (c_km1 < p).all()


def test_topp_uniform_scores_take_lowest_indices():
    # Q = 0 makes every block score 0, so all probabilities equal 1/nb exactly
    # (nb a power of two); ties go to smaller indices and k = ceil(p * nb).
    B, H, N, d, block = 1, 2, 512, 8, 64
    q = np.zeros((B, H, N, d))
    k = np.random.default_rng(4).standard_normal((B, H, N, d))
    for p in (0.3, 0.5, 0.9, 0.95):
        r = oracle.route(q, k, block, p)
        kk = math.ceil(p * 8)
        assert (r.row_cnt == kk).all()
        want = np.zeros(8, dtype=np.uint8)
        want[:kk] = 1
        assert (r.mask == want).all()


def test_topp_tiny_p_is_argmax_and_single_block_is_all():
    rng = np.random.default_rng(5)
    prob = scipy.special.softmax(rng.standard_normal((1, 2, 6, 9)) * 2, axis=-1)
    order, cum, cnt = oracle.top_p_select(prob, 1e-12)
    assert (cnt == 1).all()
    np.testing.assert_array_equal(order[..., 0], np.argmax(prob, axis=-1))
    q = rng.standard_normal((1, 2, 50, 4))
    r = oracle.route(q, q, 64, 0.5)
    assert r.mask.shape == (1, 2, 1, 1) and (r.mask == 1).all() and (r.row_cnt == 1).all()


def test_topp_p_one_selects_everything_even_underflow():
    # Scores so spread that some probabilities underflow to exactly 0.
    z = np.array([0.0, -800.0, -5.0, -2000.0])[None, None, None]
    prob = oracle.softmax_rows(z)
    assert (prob == 0).any()
    order, cum, cnt = oracle.top_p_select(prob, 1.0)
    assert (cnt == 4).all()


def test_route_end_to_end_against_brute_force():
    rng = np.random.default_rng(6)
    B, H, N, d, block = 1, 2, 70, 6, 8            # nb = 9, ragged tail of 6
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H, N, d)) + q * 0.5
    for p in (0.5, 0.9):
        r = oracle.route(q, k, block, p)
        nb = oracle.num_blocks(N, block)
        # independent recomputation of pooled scores with token loops
        for h in range(H):
            qb = [np.mean(q[0, h, i * block:min(N, (i + 1) * block)], axis=0) for i in range(nb)]
            kb = [np.mean(k[0, h, j * block:min(N, (j + 1) * block)], axis=0) for j in range(nb)]
            for i in range(nb):
                z = np.array([sum(qb[i][c] * kb[j][c] for c in range(d)) for j in range(nb)])
                z = z / math.sqrt(d)
                prob = scipy.special.softmax(z)
                want = _brute_force_topp(prob, p)
                got = set(np.nonzero(r.mask[0, h, i])[0].tolist())
                assert got == want
                assert r.row_idx[0, h, i, : len(want)].tolist() == sorted(want)
                assert (r.row_idx[0, h, i, len(want):] == -1).all()
                assert r.row_cnt[0, h, i] == len(want)
        assert (r.head_cnt == r.row_cnt.sum(-1)).all()


def test_ambiguity_window_flags_near_cut_only():
    prob = np.array([0.5, 0.3125, 0.125, 0.0625])[None, None, None]
    q = np.zeros((1, 1, 4, 2))
    r = oracle.RouteResult(q, q, prob, prob, *oracle.top_p_select(prob, 0.9)[:2],
                           oracle.top_p_select(prob, 0.9)[2], None, None, None, 0.9)
    amb = oracle.ambiguous_blocks(r, window=1e-5)
    assert not amb.any()
    prob2 = np.array([0.5, 0.3, 0.1, 0.1])[None, None, None]   # cum 0.5, 0.8, 0.9, 1.0
    order, cum, cnt = oracle.top_p_select(prob2, 0.9)
    r2 = oracle.RouteResult(q, q, prob2, prob2, order, cum, cnt, None, None, None, 0.9)
    amb2 = oracle.ambiguous_blocks(r2, window=1e-5)
    assert amb2[0, 0, 0, 2] and amb2[0, 0, 0, 3] and not amb2[0, 0, 0, 0]



def _dyadic(expr: str, eps: float) -> float:
    """Value of a fixture entry 'a', 'a + k*eps' or 'a - eps' (exact in fp64)."""
    m = re.fullmatch(r"\s*([0-9.]+)\s*(?:([+-])\s*(?:(\d+)\*)?eps)?\s*", expr)
    assert m, expr
    v = float(m.group(1))
    if m.group(2):
        k = int(m.group(3) or 1)
        v = v + k * eps if m.group(2) == "+" else v - k * eps
    return v


def test_ambiguity_swap_across_the_cut_golden(golden_dir):
    # Hand-worked rows in which no cumulative sum comes near p, so only the
    # swap-across-the-cut half of the rule can flag a block.
    g = _load(golden_dir, "ambiguity_rows.json")
    eps = 2.0 ** -18
    for case in g["cases"]:
        prob = np.array([_dyadic(s, eps) for s in case["prob"]])
        assert prob.sum() == 1.0, case["name"]
        p = case["top_p"]
        order, cum, cnt = oracle.top_p_select(prob[None, None, None], p)
        sel = sorted(order[0, 0, 0, : cnt[0, 0, 0]].tolist())
        assert sel == case["selected"], case["name"]
        excl = cum - np.take_along_axis(prob[None, None, None], order, -1)
        assert (np.abs(cum - p) >= 0.025).all() and (np.abs(excl - p) >= 0.025).all(), case["name"]
        q = np.zeros((1, 1, prob.size, 2))
        r = oracle.RouteResult(q, q, prob[None, None, None], prob[None, None, None], order, cum, cnt,
                               None, None, None, p)
        amb = oracle.ambiguous_blocks(r, window=g["window"])
        assert amb[0, 0, 0].astype(int).tolist() == case["ambiguous"], case["name"]

# ----------------------------------------------------------- causal routing ---

def test_causal_route_against_brute_force():
    # Row i: softmax over the i+1 scores j <= i only, then top-p among them.
    rng = np.random.default_rng(7)
    B, H, N, d, block = 1, 2, 70, 6, 8            # nb = 9, ragged tail of 6
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H, N, d)) + q * 0.5
    nb = oracle.num_blocks(N, block)
    for p in (0.3, 0.6, 0.9):
        r = oracle.route(q, k, block, p, causal=True)
        for h in range(H):
            qb = [np.mean(q[0, h, i * block:min(N, (i + 1) * block)], axis=0) for i in range(nb)]
            kb = [np.mean(k[0, h, j * block:min(N, (j + 1) * block)], axis=0) for j in range(nb)]
            for i in range(nb):
                z = np.array([sum(qb[i][c] * kb[j][c] for c in range(d)) for j in range(i + 1)])
                prob = scipy.special.softmax(z / math.sqrt(d))
                want = _brute_force_topp(prob, p)
                got = set(np.nonzero(r.mask[0, h, i])[0].tolist())
                assert got == want, (p, h, i)
                assert r.row_cnt[0, h, i] == len(want)
                assert r.row_idx[0, h, i, : len(want)].tolist() == sorted(want)
                np.testing.assert_allclose(r.prob[0, h, i, : i + 1], prob, rtol=1e-13, atol=0)
                assert (r.prob[0, h, i, i + 1:] == 0).all()


@pytest.mark.parametrize("p", [0.01, 0.5, 0.9, 1.0])
def test_causal_route_never_looks_ahead(p):
    rng = np.random.default_rng(8)
    q = rng.standard_normal((2, 3, 300, 4))
    k = rng.standard_normal((2, 3, 300, 4))
    r = oracle.route(q, k, 32, p, causal=True)
    nb = 10
    assert (np.triu(np.ones((nb, nb), dtype=np.uint8), 1) * r.mask == 0).all()
    assert (r.row_cnt >= 1).all() and (r.row_cnt <= np.arange(1, nb + 1)).all()
    assert (r.mask[..., 0, :] == np.eye(1, nb, 0, dtype=np.uint8)).all()      # row 0 sees block 0 only
    if p >= 1.0:                                                               # closed form: lower triangle
        assert (r.mask == np.tril(np.ones((nb, nb), dtype=np.uint8))).all()
        assert (r.head_cnt == nb * (nb + 1) // 2).all()


def test_causal_uniform_scores_take_lowest_indices():
    # Q = 0: the i+1 eligible blocks of row i tie at 1/(i+1) (exact for i+1 a
    # power of two), so k_i = ceil(p (i+1)) and the lowest indices win.
    q = np.zeros((1, 1, 512, 8))
    k = np.random.default_rng(9).standard_normal((1, 1, 512, 8))
    for p in (0.3, 0.5, 0.9):
        r = oracle.route(q, k, 64, p, causal=True)
        for i in (0, 1, 3, 7):
            kk = math.ceil(p * (i + 1))
            assert r.row_cnt[0, 0, i] == kk
            assert r.mask[0, 0, i].tolist() == [1] * kk + [0] * (8 - kk)


def test_causal_row_equals_full_routing_of_the_prefix():
    # Cutting j > i before the softmax makes row i of causal routing the same
    # as full routing of the key prefix that ends with block i.
    rng = np.random.default_rng(10)
    q = rng.standard_normal((1, 2, 200, 5))
    k = rng.standard_normal((1, 2, 200, 5))
    block, p = 16, 0.8
    rc = oracle.route(q, k, block, p, causal=True)
    for i in range(oracle.num_blocks(200, block)):
        end = min(200, (i + 1) * block)
        rf = oracle.route(q, k[:, :, :end], block, p)
        np.testing.assert_array_equal(rc.mask[:, :, i, : i + 1], rf.mask[:, :, i])
        np.testing.assert_array_equal(rc.row_cnt[:, :, i], rf.row_cnt[:, :, i])


def test_causal_ambiguity_ignores_future_blocks():
    rng = np.random.default_rng(11)
    q = rng.standard_normal((1, 2, 256, 4))
    r = oracle.route(q, q, 32, 0.7, causal=True)
    amb = oracle.ambiguous_blocks(r, window=0.5)
    assert not (amb & (np.triu(np.ones((8, 8), dtype=bool), 1))).any()
    assert amb.any()


def test_causal_executed_flops_closed_form():
    N, block, d = 200, 64, 8                      # blocks of 64, 64, 64, 8
    nb = oracle.num_blocks(N, block)
    full = np.tril(np.ones((nb, nb), dtype=np.uint8))
    assert oracle.executed_flops(full, N, block, d, causal=True) == oracle.dense_flops(1, 1, N, d, causal=True)
    assert oracle.executed_flops(np.ones((nb, nb)), N, block, d) == oracle.dense_flops(1, 1, N, d)



# ------------------------------------------------- query block != key block ---

@pytest.mark.parametrize("bq,bk", [(16, 8), (8, 16), (16, 16)])
def test_mixed_blocks_route_against_brute_force(bq, bk):
    rng = np.random.default_rng(20 + bq + bk)
    B, H, N, d = 1, 2, 70, 6                      # ragged tails for every block size
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H, N, d)) + q * 0.4
    nbq, nbk = oracle.num_blocks(N, bq), oracle.num_blocks(N, bk)
    for p in (0.5, 0.9):
        r = oracle.route(q, k, bq, p, key_block=bk)
        assert r.mask.shape == (B, H, nbq, nbk)
        for h in range(H):
            qb = [np.mean(q[0, h, i * bq:min(N, (i + 1) * bq)], axis=0) for i in range(nbq)]
            kb = [np.mean(k[0, h, j * bk:min(N, (j + 1) * bk)], axis=0) for j in range(nbk)]
            for i in range(nbq):
                z = np.array([sum(qb[i][c] * kb[j][c] for c in range(d)) for j in range(nbk)]) / math.sqrt(d)
                want = _brute_force_topp(scipy.special.softmax(z), p)
                assert set(np.nonzero(r.mask[0, h, i])[0].tolist()) == want
                assert r.row_idx[0, h, i, :len(want)].tolist() == sorted(want)


@pytest.mark.parametrize("bq,bk", [(16, 8), (8, 16), (16, 32)])
def test_mixed_blocks_causal_route_against_token_brute_force(bq, bk):
    # Key block j is eligible for query block i iff some key of j is at or
    # before some query of i, checked over token positions.
    rng = np.random.default_rng(30 + bq + bk)
    B, H, N, d = 1, 2, 75, 5
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H, N, d))
    nbq, nbk = oracle.num_blocks(N, bq), oracle.num_blocks(N, bk)
    elig = np.array([[any(s <= t for t in range(i * bq, min(N, (i + 1) * bq))
                          for s in range(j * bk, min(N, (j + 1) * bk))) for j in range(nbk)] for i in range(nbq)])
    for p in (0.6, 1.0):
        r = oracle.route(q, k, bq, p, causal=True, key_block=bk)
        assert (r.valid[0, 0] == elig.sum(1)).all()
        assert not (r.mask[0] & ~elig[None]).any()
        for h in range(H):
            qb = [np.mean(q[0, h, i * bq:min(N, (i + 1) * bq)], axis=0) for i in range(nbq)]
            kb = [np.mean(k[0, h, j * bk:min(N, (j + 1) * bk)], axis=0) for j in range(nbk)]
            for i in range(nbq):
                js = np.nonzero(elig[i])[0]
                z = np.array([sum(qb[i][c] * kb[j][c] for c in range(d)) for j in js]) / math.sqrt(d)
                want = {int(js[x]) for x in _brute_force_topp(scipy.special.softmax(z), p)}
                assert set(np.nonzero(r.mask[0, h, i])[0].tolist()) == want, (p, h, i)


@pytest.mark.parametrize("bq,bk", [(16, 8), (8, 16)])
@pytest.mark.parametrize("causal", [False, True])
def test_mixed_blocks_flops_against_token_pairs(bq, bk, causal):
    N, d = 45, 4
    nbq, nbk = oracle.num_blocks(N, bq), oracle.num_blocks(N, bk)
    mask = (np.random.default_rng(bq * bk).random((nbq, nbk)) < 0.5).astype(np.uint8)
    pairs = sum(1 for t in range(N) for s in range(N)
                if mask[t // bq, s // bk] and (not causal or s <= t))
    assert oracle.executed_flops(mask, N, bq, d, causal, key_block=bk) == 4 * d * pairs
