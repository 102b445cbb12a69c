"""Pins for the attention oracle: torch's fp64 CPU scaled_dot_product_attention
as a library special case, a naive per-query loop, a second formulation of the
mask, closed forms and invariants (no GPU)."""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle


def _sdpa(q, k, v, scale, causal=False, attn_mask=None):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    out = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=attn_mask, is_causal=causal, scale=scale)
    return out.numpy()


@pytest.mark.parametrize("shape,block,causal", [
    ((1, 2, 256, 64), 64, False),
    ((1, 2, 256, 64), 64, True),
    ((2, 3, 77, 16), 16, False),
    ((2, 3, 77, 16), 16, True),
    ((1, 1, 130, 32), 128, True),
])
def test_dense_matches_torch_sdpa_fp64(shape, block, causal):
    rng = np.random.default_rng(sum(shape) + block + causal)
    q, k, v = (rng.standard_normal(shape) for _ in range(3))
    scale = 1 / math.sqrt(shape[-1])
    o, lse = oracle.attend(q, k, v, block, mask=None, scale=scale, causal=causal)
    np.testing.assert_allclose(o, _sdpa(q, k, v, scale, causal), rtol=1e-12, atol=1e-12)
    logits = scale * np.einsum("bhqd,bhkd->bhqk", q, k)
    if causal:
        n = shape[2]
        logits = np.where(np.tril(np.ones((n, n), dtype=bool)), logits, -np.inf)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(logits, axis=-1), rtol=1e-13, atol=1e-13)


def test_dense_matches_naive_per_query_loop():
    rng = np.random.default_rng(7)
    N, d, block = 11, 3, 4
    q, k, v = (rng.standard_normal((1, 1, N, d)) for _ in range(3))
    o, lse = oracle.attend(q, k, v, block, scale=0.7)
    for t in range(N):
        logits = [0.7 * sum(q[0, 0, t, c] * k[0, 0, s, c] for c in range(d)) for s in range(N)]
        mu = max(logits)
        w = [math.exp(x - mu) for x in logits]
        den = math.fsum(w)
        for c in range(d):
            assert abs(o[0, 0, t, c] - math.fsum(w[s] * v[0, 0, s, c] for s in range(N)) / den) < 1e-13
        assert abs(lse[0, 0, t] - (mu + math.log(den))) < 1e-13


def _random_mask(rng, B, H, nb):
    m = (rng.random((B, H, nb, nb)) < 0.4).astype(np.uint8)
    m[..., np.arange(nb), rng.integers(0, nb, size=nb)] = 1       # every row selects >= 1 block
    return m


@pytest.mark.parametrize("causal", [False, True])
def test_gather_form_equals_masked_logit_form(causal):
    rng = np.random.default_rng(8)
    B, H, N, d, block = 1, 2, 90, 8, 16                          # ragged tail of 10
    q, k, v = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    nb = oracle.num_blocks(N, block)
    mask = _random_mask(rng, B, H, nb)
    if causal:
        mask[..., np.arange(nb), np.arange(nb)] = 1               # diagonal keeps each query non-empty
    o1, l1 = oracle.attend(q, k, v, block, mask=mask, causal=causal)
    o2, l2 = oracle.attend_dense_masked_logits(q, k, v, block, mask=mask, causal=causal)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=1e-13, atol=1e-13)


def test_masked_rows_equal_sdpa_on_gathered_keys():
    # Reduction to dense: a masked query block equals plain attention over
    # the concatenated tokens of its selected key blocks.
    rng = np.random.default_rng(9)
    B, H, N, d, block = 1, 1, 100, 16, 32
    q, k, v = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    nb = oracle.num_blocks(N, block)
    mask = _random_mask(rng, B, H, nb)
    o, _ = oracle.attend(q, k, v, block, mask=mask, scale=0.25)
    for i in range(nb):
        keys = np.concatenate([np.arange(j * block, min(N, (j + 1) * block))
                               for j in np.nonzero(mask[0, 0, i])[0]])
        rows = slice(i * block, min(N, (i + 1) * block))
        want = _sdpa(q[:, :, rows], k[:, :, keys], v[:, :, keys], 0.25)
        np.testing.assert_allclose(o[:, :, rows], want, rtol=1e-12, atol=1e-12)


def test_p_one_route_gives_dense_exactly():
    rng = np.random.default_rng(10)
    shape = (1, 2, 256, 64)
    q, k, v = (rng.standard_normal(shape) for _ in range(3))
    r = oracle.route(q, k, 64, 1.0)
    assert (r.mask == 1).all()
    o_s, l_s = oracle.attend(q, k, v, 64, mask=r.mask)
    o_d, l_d = oracle.attend(q, k, v, 64, mask=None)
    np.testing.assert_array_equal(o_s, o_d)
    np.testing.assert_array_equal(l_s, l_d)


def test_closed_forms_constant_v_constant_k_dominant_key():
    rng = np.random.default_rng(11)
    B, H, N, d, block = 1, 1, 96, 8, 32
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H, N, d))
    nb = oracle.num_blocks(N, block)
    mask = _random_mask(rng, B, H, nb)
    # V constant -> O constant.
    v = np.full((B, H, N, d), 0.375)
    o, _ = oracle.attend(q, k, v, block, mask=mask)
    np.testing.assert_allclose(o, 0.375, rtol=0, atol=1e-15)
    # K constant -> uniform weights: O = mean of V over the allowed keys, LSE = l + ln|A|.
    v = rng.standard_normal((B, H, N, d))
    kc = np.broadcast_to(rng.standard_normal(d), (B, H, N, d)).copy()
    o, lse = oracle.attend(q, kc, v, block, mask=mask, scale=0.5)
    for i in range(nb):
        keys = np.concatenate([np.arange(j * block, min(N, (j + 1) * block))
                               for j in np.nonzero(mask[0, 0, i])[0]])
        rows = np.arange(i * block, min(N, (i + 1) * block))
        np.testing.assert_allclose(o[0, 0, rows], np.broadcast_to(v[0, 0, keys].mean(0), (rows.size, d)),
                                   rtol=1e-12, atol=1e-12)
        lvals = 0.5 * q[0, 0, rows] @ kc[0, 0, 0]
        np.testing.assert_allclose(lse[0, 0, rows], lvals + math.log(keys.size), rtol=1e-12, atol=1e-12)
    # One key far above the rest -> O is that key's value row.
    q1 = np.zeros((B, H, N, d)); q1[..., 0] = 1.0
    k1 = np.zeros((B, H, N, d)); k1[0, 0, 40, 0] = 2000.0
    full = np.ones((B, H, nb, nb), dtype=np.uint8)
    o, _ = oracle.attend(q1, k1, v, block, mask=full, scale=1.0)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0, 0, 40], (N, d)), rtol=0, atol=1e-12)


def test_weights_sum_to_one_via_lse():
    rng = np.random.default_rng(12)
    B, H, N, d, block = 1, 1, 64, 4, 16
    q, k = (rng.standard_normal((B, H, N, d)) * 3 for _ in range(2))
    v = np.eye(N)[None, None, :, :d] * 0 + 1.0
    _, lse = oracle.attend(q, k, v, block, scale=1.0, causal=True)
    logits = q[0, 0] @ k[0, 0].T
    for t in range(N):
        w = np.exp(logits[t, : t + 1] - lse[0, 0, t])
        assert abs(w.sum() - 1.0) < 1e-13 and (w >= 0).all()



@pytest.mark.parametrize("bq,bk", [(16, 32), (32, 16)])
@pytest.mark.parametrize("causal", [False, True])
def test_mixed_blocks_gather_equals_masked_logits(bq, bk, causal):
    rng = np.random.default_rng(40 + bq)
    q, k, v = (rng.standard_normal((1, 2, 90, 8)) for _ in range(3))
    nbq, nbk = -(-90 // bq), -(-90 // bk)
    mask = (rng.random((1, 2, nbq, nbk)) < 0.6).astype(np.uint8)
    mask[..., 0] = 1                               # every query keeps at least key block 0
    o1, l1 = oracle.attend(q, k, v, bq, mask=mask, causal=causal, key_block=bk)
    o2, l2 = oracle.attend_dense_masked_logits(q, k, v, bq, mask=mask, causal=causal, key_block=bk)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)



def test_queries_without_allowed_keys_get_zero_and_neg_inf():
    # Causal attention with query blocks of 32 over key blocks of 16: query
    # block 1 (tokens 32..63) listing only key block 3 (tokens 48..63) leaves
    # tokens 32..47 without keys; tokens 48..63 see keys 48..t.
    rng = np.random.default_rng(50)
    q, k, v = (rng.standard_normal((1, 1, 64, 4)) for _ in range(3))
    mask = np.zeros((1, 1, 2, 4), dtype=np.uint8)
    mask[0, 0, 0, 0] = 1
    mask[0, 0, 1, 3] = 1
    o, lse = oracle.attend(q, k, v, 32, mask=mask, causal=True, key_block=16)
    assert (o[0, 0, 32:48] == 0).all() and np.isneginf(lse[0, 0, 32:48]).all()
    for t in range(48, 64):
        keys = np.arange(48, t + 1)
        lg = (q[0, 0, t] @ k[0, 0, keys].T) / 2.0
        w = np.exp(lg - lg.max())
        np.testing.assert_allclose(o[0, 0, t], (w @ v[0, 0, keys]) / w.sum(), rtol=1e-12, atol=1e-13)
    o2, lse2 = oracle.attend_dense_masked_logits(q, k, v, 32, mask=mask, causal=True, key_block=16)
    np.testing.assert_array_equal(o2[0, 0, 32:48], 0.0)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-12)
    assert (np.isneginf(lse2) == np.isneginf(lse)).all()
