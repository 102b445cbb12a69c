"""Block-masked softmax attention in float64 (oracle; test infrastructure only).

Source: FlashAttention review page, Background [3] (Motivation): S = Q K^T,
P = softmax(S), O = P V; the Introduction states FlashAttention is exact, so
its output is this plain result.  The top-p mask of the FVAttn review page
(section 1, "Top-p routing") restricts, for every query of query block i, the
keys to the tokens of the key blocks selected for row i.  Unselected keys are
excluded from the softmax (renormalised over the allowed keys).  With
`causal`, a query at position t additionally sees only keys at positions <= t.

For each query t with allowed key set A_t and logits l_s = scale * <Q_t, K_s>:
    mu    = max_{s in A_t} l_s
    O_t   = sum_{s in A_t} exp(l_s - mu) V_s / sum_{s in A_t} exp(l_s - mu)
    LSE_t = mu + ln sum_{s in A_t} exp(l_s - mu)          (natural log)
A query with no allowed key (empty A_t: no selected key block, or, under a
causal mask, selected key blocks that all start after it) gets O_t = 0 and
LSE_t = -inf, the values of the empty sums; the pages leave this case open.
"""
from __future__ import annotations

import numpy as np

from .routing import num_blocks


def _allowed_keys(mask_row, n_tokens: int, block: int) -> np.ndarray:
    """Token indices of the selected key blocks, ascending."""
    sel = np.nonzero(mask_row)[0]
    if sel.size == 0:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate([np.arange(j * block, min(n_tokens, (j + 1) * block)) for j in sel])


def _attend_rows(q_rows, q_pos, k_h, v_h, keys, scale, causal):
    """Attention of a few query rows over an explicit key index set."""
    n = q_rows.shape[0]
    if keys.size == 0:
        return np.zeros((n, v_h.shape[1])), np.full(n, -np.inf)
    kk = k_h[keys]
    vv = v_h[keys]
    logits = scale * (q_rows @ kk.T)
    if causal:
        logits = np.where(keys[None, :] <= q_pos[:, None], logits, -np.inf)
    has = np.isfinite(logits).any(axis=1)                  # rows with at least one allowed key
    mu = np.max(np.where(has[:, None], logits, 0.0), axis=1, keepdims=True)
    w = np.exp(logits - mu)
    denom = np.sum(w, axis=1, keepdims=True)
    out = np.where(has[:, None], (w @ vv) / np.where(has[:, None], denom, 1.0), 0.0)
    lse = np.where(has, mu[:, 0] + np.log(np.where(has, denom[:, 0], 1.0)), -np.inf)
    return out, lse


def attend_units(q, k, v, block: int, units, mask=None, scale: float | None = None,
                 causal: bool = False, key_block: int | None = None):
    """Attention output of selected query blocks.

    q, k, v: [B, H, N, d]; units: iterable of (b, h, i) with i a query block of
    `block` tokens; mask: [B, H, nbq, nbk] block mask over key blocks of
    `key_block` tokens (default: block; None means every key block).  Returns
    {(b, h, i): (O, LSE)} with O of shape [n_i, d] and LSE of shape [n_i],
    both float64.
    """
    kb = block if key_block is None else key_block
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, d = q.shape
    nbk = num_blocks(N, kb)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = {}
    for (b, h, i) in units:
        lo, hi = i * block, min(N, (i + 1) * block)
        row = np.ones(nbk, dtype=np.uint8) if mask is None else mask[b, h, i]
        keys = _allowed_keys(row, N, kb)
        q_pos = np.arange(lo, hi)
        out[(b, h, i)] = _attend_rows(q[b, h, lo:hi], q_pos, k[b, h], v[b, h], keys,
                                      scale, causal)
    return out


def attend(q, k, v, block: int, mask=None, scale: float | None = None, causal: bool = False,
           key_block: int | None = None):
    """Full output O [B, H, N, d] and LSE [B, H, N] (float64)."""
    q64 = np.asarray(q, dtype=np.float64)
    B, H, N, d = q64.shape
    nb = num_blocks(N, block)
    units = [(b, h, i) for b in range(B) for h in range(H) for i in range(nb)]
    res = attend_units(q64, k, v, block, units, mask=mask, scale=scale, causal=causal, key_block=key_block)
    o = np.empty((B, H, N, d), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    for (b, h, i), (ob, lb) in res.items():
        lo, hi = i * block, min(N, (i + 1) * block)
        o[b, h, lo:hi] = ob
        lse[b, h, lo:hi] = lb
    return o, lse


def attend_dense_masked_logits(q, k, v, block: int, mask=None, scale: float | None = None,
                               causal: bool = False, key_block: int | None = None):
    """Same result as `attend`, written as one full logit matrix per head with
    -inf at disallowed (query, key) pairs.  A second formulation used to pin
    the gather form above; O(N^2) memory, small inputs only."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    tok_blk = np.arange(N) // block
    key_blk = np.arange(N) // (block if key_block is None else key_block)
    o = np.empty_like(q)
    lse = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            logits = scale * (q[b, h] @ k[b, h].T)
            allowed = np.ones((N, N), dtype=bool)
            if mask is not None:
                allowed &= mask[b, h][tok_blk[:, None], key_blk[None, :]].astype(bool)
            if causal:
                allowed &= np.arange(N)[None, :] <= np.arange(N)[:, None]
            logits = np.where(allowed, logits, -np.inf)
            has = allowed.any(axis=1)
            mu = np.where(has[:, None], logits, 0.0).max(axis=1, keepdims=True)
            w = np.exp(logits - mu)
            den = w.sum(axis=1, keepdims=True)
            o[b, h] = np.where(has[:, None], (w @ v[b, h]) / np.where(has[:, None], den, 1.0), 0.0)
            lse[b, h] = np.where(has, mu[:, 0] + np.log(np.where(has, den[:, 0], 1.0)), -np.inf)
    return o, lse
