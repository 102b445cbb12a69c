"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch each one: a transposed operand, a wrong divisor, an exclusive threshold,
a reversed tie rule, a dropped scale, an off-by-one causal mask, a wrong log
base, a wrong sort direction, and a causal block cut that is missing, off by
one, or applied after the softmax instead of before it; and an augmentation
that takes the lowest-probability candidates, measures slack from the mean
load, or draws candidates from every worker's rows; an E4M3 exponent bias off by
one, ties rounded away from zero, K scaled per token instead of per tile, and
an inverted dequantisation scale."""
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


def test_sasa_lowest_probability_first_caught(monkeypatch):
    orig = sa.augment

    def low_first(prob, *a, **k):
        return orig(-np.asarray(prob), *a, **k)
    monkeypatch.setattr(oracle, "augment", low_first)
    with pytest.raises(AssertionError):
        ts.test_brute_force_added_blocks_carry_max_mass(0, 400, 1, 6)


def test_sasa_slack_from_mean_caught(monkeypatch):
    orig_lpt = sa.lpt_assign

    def mean_makespan(costs, order, W):
        worker_of, load = orig_lpt(costs, order, W)
        # a wrong slack: measured from the mean load (raise every load to the max minus the mean)
        return worker_of, load - (load.max() - int(load.mean()))
    monkeypatch.setattr(sa, "lpt_assign", mean_makespan)
    with pytest.raises(AssertionError):
        ts.test_hand_example_two_workers()


def test_sasa_candidates_from_all_rows_caught(monkeypatch):
    orig_lpt = sa.lpt_assign

    def one_worker_rows(costs, order, W):
        worker_of, load = orig_lpt(costs, order, W)
        return np.zeros_like(worker_of), load          # every row counted as worker 0's
    monkeypatch.setattr(sa, "lpt_assign", one_worker_rows)
    with pytest.raises(AssertionError):
        ts.test_hand_example_three_workers_ties()


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
