"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch each one: a transposed operand, a wrong divisor, an exclusive threshold,
a reversed tie rule, a dropped scale, an off-by-one causal mask, a wrong log
base, a wrong sort direction, and a causal block cut that is missing, off by
one, or applied after the softmax instead of before it; an augmentation that
buys the lowest-value pairs, breaks ties the wrong way, drops the fixed cost
of a tile, charges it for every pair, passes over a pair it cannot afford
instead of stopping, assigns items with the sequential LPT, spends slack on
a worker's first item, prices items in union tiles only, or prices a key
block as one tile; an E4M3 exponent bias off by
one, ties rounded away from zero, K scaled per token instead of per tile, and
an inverted dequantisation scale; and an ambiguity window whose swap-across-
the-cut rule is dropped (whole or either half), measured against the wrong
neighbour, or applied to near ties between any two neighbouring ranks."""
import numpy as np
import pytest

import oracle
import oracle.attention as att
import oracle.routing as rt
import oracle.sasa as sa
import test_oracle_attention as ta
import test_oracle_routing as tr
import test_oracle_sasa as ts


def _patch(monkeypatch, module, name, fn):
    monkeypatch.setattr(module, name, fn)
    if hasattr(oracle, name):
        monkeypatch.setattr(oracle, name, fn)


def test_transposed_scores_caught(monkeypatch, golden_dir):
    orig = rt.block_scores
    _patch(monkeypatch, rt, "block_scores", lambda q, k, s: orig(k, q, s))
    with pytest.raises(AssertionError):
        tr.test_pool_and_scores_hand_example(golden_dir)


def test_pool_divisor_caught(monkeypatch):
    def bad_pool(x, block):
        x = np.asarray(x, dtype=np.float64)
        B, H, N, d = x.shape
        nb = rt.num_blocks(N, block)
        out = np.empty((B, H, nb, d))
        for i in range(nb):
            out[:, :, i] = x[:, :, i * block:(i + 1) * block].sum(axis=2) / block
        return out
    _patch(monkeypatch, rt, "pool_blocks", bad_pool)
    with pytest.raises(AssertionError):
        tr.test_pool_constant_blocks_with_ragged_tail()


def test_exclusive_threshold_caught(monkeypatch, golden_dir):
    orig = rt.top_p_select

    def strict(prob, p, valid=None):
        order, cum, cnt = orig(prob, p, valid)
        if p < 1:
            reached = cum > p
            cnt = np.where(reached.any(-1), np.argmax(reached, -1) + 1, prob.shape[-1])
        return order, cum, cnt
    _patch(monkeypatch, rt, "top_p_select", strict)
    with pytest.raises(AssertionError):
        tr.test_topp_golden_rows(golden_dir)


def test_reversed_tie_rule_caught(monkeypatch):
    def rev_ties(prob, p, valid=None):
        nb = prob.shape[-1]
        flipped = prob[..., ::-1]
        order = nb - 1 - np.argsort(-flipped, axis=-1, kind="stable")
        ranked = np.take_along_axis(prob, order, -1)
        cum = np.cumsum(ranked, -1)
        reached = cum >= p
        cnt = np.where(reached.any(-1), np.argmax(reached, -1) + 1, nb) if p < 1 else np.full(prob.shape[:-1], nb)
        return order, cum, cnt
    _patch(monkeypatch, rt, "top_p_select", rev_ties)
    with pytest.raises(AssertionError):
        tr.test_topp_uniform_scores_take_lowest_indices()


def test_ascending_sort_caught(monkeypatch):
    def ascending(prob, p, valid=None):
        nb = prob.shape[-1]
        order = np.argsort(prob, axis=-1, kind="stable")
        cum = np.cumsum(np.take_along_axis(prob, order, -1), -1)
        reached = cum >= p
        cnt = np.where(reached.any(-1), np.argmax(reached, -1) + 1, nb) if p < 1 else np.full(prob.shape[:-1], nb)
        return order, cum, cnt
    _patch(monkeypatch, rt, "top_p_select", ascending)
    with pytest.raises(AssertionError):
        tr.test_topp_brute_force_subsets(7, 0.5)


def test_dropped_scale_caught(monkeypatch):
    orig = att._attend_rows
    monkeypatch.setattr(att, "_attend_rows", lambda qr, qp, k, v, keys, s, c: orig(qr, qp, k, v, keys, 1.0, c))
    with pytest.raises(AssertionError):
        ta.test_dense_matches_torch_sdpa_fp64((1, 2, 256, 64), 64, False)


def test_causal_off_by_one_caught(monkeypatch):
    def strict_causal(q_rows, q_pos, k_h, v_h, keys, scale, causal):
        kk, vv = k_h[keys], v_h[keys]
        logits = scale * (q_rows @ kk.T)
        if causal:
            logits = np.where(keys[None, :] < q_pos[:, None], logits, -np.inf)
        mu = np.max(logits, axis=1, keepdims=True)
        mu = np.where(np.isfinite(mu), mu, 0.0)
        w = np.exp(logits - mu)
        den = np.sum(w, axis=1, keepdims=True)
        return (w @ vv) / den, mu[:, 0] + np.log(den[:, 0])
    monkeypatch.setattr(att, "_attend_rows", strict_causal)
    with pytest.raises(AssertionError):
        ta.test_dense_matches_torch_sdpa_fp64((2, 3, 77, 16), 16, True)


def test_wrong_log_base_caught(monkeypatch):
    orig = att._attend_rows

    def log2_lse(*a):
        o, lse = orig(*a)
        return o, lse / np.log(2.0)
    monkeypatch.setattr(att, "_attend_rows", log2_lse)
    with pytest.raises(AssertionError):
        ta.test_dense_matches_torch_sdpa_fp64((1, 2, 256, 64), 64, False)


def test_missing_causal_cut_caught(monkeypatch):
    _patch(monkeypatch, rt, "causal_cut", lambda z, valid=None: z)
    with pytest.raises(AssertionError):
        tr.test_causal_route_never_looks_ahead(0.5)


def test_causal_cut_off_by_one_caught(monkeypatch):
    def late_cut(z, valid=None):
        nb = z.shape[-1]
        ahead = np.arange(nb)[None, :] > np.arange(nb)[:, None] + 1
        return np.where(ahead, -np.inf, z)
    _patch(monkeypatch, rt, "causal_cut", late_cut)
    with pytest.raises(AssertionError):
        tr.test_causal_route_never_looks_ahead(0.9)


def test_causal_cut_after_softmax_caught(monkeypatch):
    # zero the future probabilities after a full softmax, without renormalising
    orig = rt.softmax_rows

    def cut_after(z):
        prob = orig(z)
        nb = z.shape[-1]
        return np.where(np.arange(nb)[None, :] > np.arange(nb)[:, None], 0.0, prob)
    _patch(monkeypatch, rt, "causal_cut", lambda z, valid=None: z)
    _patch(monkeypatch, rt, "softmax_rows", cut_after)
    with pytest.raises(AssertionError):
        tr.test_causal_route_against_brute_force()


def test_sasa_lowest_value_first_caught(monkeypatch):
    monkeypatch.setattr(sa, "buy_order", lambda value, row, j: (value, row, j))
    with pytest.raises(AssertionError):
        ts.test_purchase_is_the_longest_affordable_prefix(1, 400, 2, 5, False, 64, 3)


def test_sasa_reversed_tie_rule_caught(monkeypatch, golden_dir):
    monkeypatch.setattr(sa, "buy_order", lambda value, row, j: (-value, -row, -j))
    with pytest.raises(AssertionError):
        ts.test_golden_slack_purchase_example(golden_dir)


def test_sasa_fixed_tile_cost_dropped_caught(monkeypatch):
    monkeypatch.setattr(sa, "pair_cost", lambda tiles_j, opens, tile_fixed: tiles_j)
    with pytest.raises(AssertionError):
        ts.test_purchase_is_the_longest_affordable_prefix(1, 400, 2, 5, False, 64, 3)


def test_sasa_every_pair_opens_a_tile_caught(monkeypatch, golden_dir):
    monkeypatch.setattr(sa, "pair_cost", lambda tiles_j, opens, tile_fixed: tiles_j * (1 + tile_fixed))
    with pytest.raises(AssertionError):
        ts.test_golden_slack_purchase_example(golden_dir)


def test_sasa_skips_instead_of_stopping_caught(monkeypatch, golden_dir):
    # a purchase that passes over a pair it cannot afford and goes on
    orig_cost = sa.pair_cost
    orig_augment = sa.augment

    def patched(prob, mask, order, work_order, valid, group, W, n_tokens, key_block, tile_fixed):
        prob = np.asarray(prob, dtype=np.float64)
        mask0 = np.asarray(mask).astype(np.uint8)
        res = orig_augment(prob, mask0, order, work_order, valid, group, W, n_tokens, key_block, tile_fixed)
        B, H, nb, nbk = mask0.shape
        ng = -(-nb // group)
        tiles = sa.block_tiles(nbk, n_tokens, key_block)
        union = sa.item_unions(mask0, group)
        new = mask0.copy()
        for w in range(W):
            g = int(res.last_item[w])
            if g < 0 or res.slack[w] <= 0:
                continue
            bh, gi = divmod(g, ng)
            b, h = divmod(bh, H)
            cands = sorted(((i, j) for i in range(gi * group, min(nb, (gi + 1) * group)) for j in range(nbk)
                            if not mask0[b, h, i, j]), key=lambda c: (-prob[b, h, c[0], c[1]], c[0], c[1]))
            opened, spent = union[g].copy(), 0
            for i, j in cands:
                c = orig_cost(int(tiles[j]), not opened[j], tile_fixed)
                if spent + c <= res.slack[w]:
                    spent += c
                    opened[j] = True
                    new[b, h, i, j] = 1
        res.mask = new
        return res
    monkeypatch.setattr(oracle, "augment", patched)
    with pytest.raises(AssertionError):
        ts.test_golden_slack_purchase_example(golden_dir)


def test_sasa_sequential_lpt_caught(monkeypatch, golden_dir):
    def sequential(costs, order, W):
        worker_of, load = oracle.lpt_assign(costs, order, W)
        last = np.full(W, -1, dtype=np.int64)
        for g in order:
            last[worker_of[g]] = g
        return worker_of, load, last
    monkeypatch.setattr(sa, "lpt_batched", sequential)
    with pytest.raises(AssertionError):
        ts.test_golden_slack_purchase_example(golden_dir)


def test_sasa_slack_on_first_item_caught(monkeypatch):
    orig = sa.lpt_batched

    def first_item(costs, order, W):
        worker_of, load, _ = orig(costs, order, W)
        first = np.full(W, -1, dtype=np.int64)
        for g in reversed(np.asarray(order).tolist()):
            first[worker_of[g]] = g
        return worker_of, load, first
    monkeypatch.setattr(sa, "lpt_batched", first_item)
    with pytest.raises(AssertionError):
        ts.test_assignment_unchanged_and_makespan_kept(4, 64, 1000, 3, False)


def test_sasa_items_priced_in_union_tiles_only_caught(monkeypatch, golden_dir):
    monkeypatch.setattr(sa, "item_costs", lambda mask, group, n_tokens, key_block, tile_fixed: (
        sa.item_unions(mask, group) * sa.block_tiles(np.asarray(mask).shape[-1], n_tokens, key_block)).sum(-1))
    with pytest.raises(AssertionError):
        ts.test_golden_slack_purchase_example(golden_dir)


def test_sasa_blocks_priced_as_one_tile_caught(monkeypatch):
    # every key block priced at one tile, the kernel's 128-key blocks included
    monkeypatch.setattr(sa, "block_tiles", lambda nbk, n_tokens, key_block: np.ones(nbk, dtype=np.int64))
    with pytest.raises(AssertionError):
        ts.test_purchase_is_the_longest_affordable_prefix(2, 1064, 4, 7, False, 128, 3)


def test_mixed_block_eligibility_off_by_one_caught(monkeypatch):
    # a key block counted eligible only when it ends (not starts) before the query block's last token
    def strict(nbq, nbk, block, key_block):
        last = (np.arange(nbq, dtype=np.int64) + 1) * block - 1
        return np.maximum(1, np.minimum(nbk, (last + 1) // key_block))
    _patch(monkeypatch, rt, "causal_eligible", strict)
    with pytest.raises(AssertionError):
        tr.test_mixed_blocks_causal_route_against_token_brute_force(8, 16)


def test_union_fill_wrong_group_caught(monkeypatch):
    orig = sa.union_fill
    monkeypatch.setattr(oracle, "union_fill", lambda mask, order, valid, group: orig(mask, order, valid, 2 * group))
    with pytest.raises(AssertionError):
        ts.test_union_fill_against_brute_force(2, False)


# ------------------------------------------------------------------ fp8 ---

import oracle.fp8 as f8        # noqa: E402
import test_oracle_fp8 as tf   # noqa: E402


def test_e4m3_exponent_bias_off_by_one_caught(monkeypatch):
    orig = f8.e4m3_value
    monkeypatch.setattr(f8, "e4m3_value", lambda c: orig(c) * 2.0)
    with pytest.raises(AssertionError):
        tf.test_e4m3_closed_form_codes()


def test_e4m3_ties_away_from_zero_caught(monkeypatch, golden_dir):
    monkeypatch.setattr(f8, "_round_half_even", lambda x: np.floor(x + 0.5))
    with pytest.raises(AssertionError):
        tf.test_quantize_hand_example(golden_dir)
    with pytest.raises(AssertionError):
        tf.test_e4m3_encode_matches_torch_rounding()


def test_k_scaled_per_token_caught(monkeypatch):
    def per_token(k, tile=f8.QUANT_TILE):
        k = np.asarray(k, dtype=np.float64)
        amax = np.abs(k).max(axis=-1)
        return f8.quantize_groups(k, amax[..., None]), f8.group_factors(amax[:, :, ::tile])[1].astype(np.float32)
    monkeypatch.setattr(f8, "quantize_k", per_token)
    with pytest.raises(AssertionError):
        tf.test_quantize_group_scaling_and_locality()


def test_scale_inverted_caught(monkeypatch, golden_dir):
    orig = f8.group_factors
    monkeypatch.setattr(f8, "group_factors", lambda a: (orig(a)[0], orig(a)[0]))
    with pytest.raises(AssertionError):
        tf.test_quantize_hand_example(golden_dir)


# --------------------------------------------------- ambiguity window ---

def _ambiguity_variant(swap_in_ref="first_out", swap_out_ref="last_in", adjacent=False):
    """ambiguous_blocks with its swap rule changed: the selected blocks
    measured against `swap_in_ref` and the unselected ones against
    `swap_out_ref` (None drops that half), or (adjacent=True) any two
    neighbouring ranks within the window flagged wherever they are."""
    def amb(res, window=1e-5):
        prob, order, cum = res.prob, res.order, res.cum
        shape, nb = prob.shape, prob.shape[-1]
        if res.top_p >= 1.0:
            return np.zeros(shape, dtype=bool)
        k = np.asarray(res.row_cnt)
        valid = np.full(k.shape, nb, dtype=np.int64) if res.valid is None else np.asarray(res.valid)
        ranked = np.take_along_axis(prob, order, axis=-1)
        ref = {"last_in": np.take_along_axis(ranked, (k - 1)[..., None], axis=-1),
               "first_out": np.where((k < valid)[..., None],
                                     np.take_along_axis(ranked, np.minimum(k, nb - 1)[..., None], axis=-1),
                                     -np.inf)}
        excl = cum - ranked
        near_ranked = (np.abs(excl - res.top_p) <= window) | (np.abs(cum - res.top_p) <= window)
        near = np.zeros(shape, dtype=bool)
        np.put_along_axis(near, order, near_ranked, axis=-1)
        rank_of = np.empty_like(order)
        np.put_along_axis(rank_of, order, np.broadcast_to(np.arange(nb), shape), axis=-1)
        selected = rank_of < k[..., None]
        eligible = np.arange(nb) < valid[..., None]
        out = near & eligible
        if adjacent:
            close = np.zeros(shape, dtype=bool)
            gap = np.abs(np.diff(ranked, axis=-1)) <= window
            close_ranked = np.zeros(shape, dtype=bool)
            close_ranked[..., :-1] |= gap
            close_ranked[..., 1:] |= gap
            np.put_along_axis(close, order, close_ranked, axis=-1)
            return out | (close & eligible)
        if swap_in_ref is not None:
            out |= selected & (np.abs(prob - ref[swap_in_ref]) <= window)
        if swap_out_ref is not None:
            out |= ~selected & eligible & (np.abs(ref[swap_out_ref] - prob) <= window)
        return out
    return amb


@pytest.mark.parametrize("variant", [
    dict(swap_in_ref=None, swap_out_ref=None),            # swap rule dropped
    dict(swap_in_ref=None),                               # selected half dropped
    dict(swap_out_ref=None),                              # unselected half dropped
    dict(swap_in_ref="last_in", swap_out_ref="first_out"),  # each half against its own side of the cut
    dict(swap_out_ref="first_out"),                       # unselected blocks against the first unselected one
    dict(adjacent=True),                                  # any near tie between neighbouring ranks
])
def test_ambiguity_swap_rule_mutants_caught(monkeypatch, golden_dir, variant):
    _patch(monkeypatch, rt, "ambiguous_blocks", _ambiguity_variant(**variant))
    with pytest.raises(AssertionError):
        tr.test_ambiguity_swap_across_the_cut_golden(golden_dir)


def test_ambiguity_variant_helper_is_faithful(golden_dir):
    # The unmutated helper reproduces the oracle, so each mutant above differs
    # from it by exactly the change it names.
    tr.test_ambiguity_swap_across_the_cut_golden(golden_dir)
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 2, 512, 4))
    for p in (0.3, 0.7, 0.9):
        r = oracle.route(q, q + 0.1 * rng.standard_normal(q.shape), 16, p)
        for w in (1e-5, 1e-3, 3e-2):
            np.testing.assert_array_equal(_ambiguity_variant()(r, w), oracle.ambiguous_blocks(r, w))
