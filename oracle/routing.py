"""Top-p block routing in float64 (oracle; test infrastructure only).

Source: FVAttn review page, section 1 (Key Terms, "Top-p routing"): for each
query block, key blocks are chosen by importance score until the cumulative
probability reaches a threshold p; section 3 (Method) applies this routing
before load balancing.  The page leaves the importance score undefined; the
reading used here is the plainest one consistent with a "pool" router:

  1. nb = ceil(N / block); block i holds tokens [i*block, min((i+1)*block, N)),
     n_i of them (the last block may be short).
  2. Qbar_i = mean of Q over the n_i valid tokens of block i; Kbar_j likewise.
  3. Z_ij = scale * <Qbar_i, Kbar_j>, scale = 1/sqrt(d) unless given.
  4. P_i. = softmax over j of Z_i. .
  5. Rank j by P_ij descending, equal probabilities by smaller j first;
     C_r = sum of the first r ranked probabilities (r = 1..nb).
  6. k_i = smallest r with C_r >= p ("reaches p" read as inclusive); k_i = nb
     when p >= 1 (dense attention is the p = 1 case) or when no r qualifies.
  7. The first k_i ranked blocks are selected: mask M_ij = 1, the selected
     indices listed in ascending order, row count k_i, head count sum_i k_i.

Causal routing (the decoder setting; the page's routing is stated for
encoder-style full attention, and the block-level causal cut is the reading
taken for causal models): key blocks after the query block (j > i) are cut
before the softmax (Z_ij = -inf, so P_ij = 0 and the softmax runs over the
i+1 blocks j <= i), and "all blocks" in step 6 means those i+1 blocks.  The
attention of a causal model additionally keeps only keys s <= t for query t
(attention.attend with causal=True).

Query and key blocks may differ in size (block for queries, key_block for
keys): Qbar pools query blocks of `block` tokens, Kbar key blocks of
`key_block` tokens, and Z, P, the ranking and the selection run over the
nbk = ceil(N / key_block) key blocks of every query block.  Under causal
routing key block j is eligible for query block i when it starts at or
before the last token of query block i (j * key_block <= (i+1) * block - 1);
with equal sizes that is j <= i.
"""
from __future__ import annotations

import dataclasses

import numpy as np


def num_blocks(n_tokens: int, block: int) -> int:
    return -(-n_tokens // block)


def block_sizes(n_tokens: int, block: int) -> np.ndarray:
    """n_i: number of valid tokens in each block (int64, length nb)."""
    nb = num_blocks(n_tokens, block)
    starts = np.arange(nb, dtype=np.int64) * block
    return np.minimum(block, n_tokens - starts)


def pool_blocks(x: np.ndarray, block: int) -> np.ndarray:
    """Mean of x over the valid tokens of each block.

    x: [B, H, N, d] float64  ->  [B, H, nb, d] float64.
    """
    x = np.asarray(x, dtype=np.float64)
    B, H, N, d = x.shape
    nb = num_blocks(N, block)
    out = np.empty((B, H, nb, d), dtype=np.float64)
    for i in range(nb):
        lo, hi = i * block, min(N, (i + 1) * block)
        out[:, :, i, :] = x[:, :, lo:hi, :].sum(axis=2) / (hi - lo)
    return out


def block_scores(qbar: np.ndarray, kbar: np.ndarray, scale: float) -> np.ndarray:
    """Z = scale * Qbar Kbar^T per (b, h): [B, H, nbq, nbk]."""
    return scale * np.matmul(qbar, np.swapaxes(kbar, -1, -2))


def softmax_rows(z: np.ndarray) -> np.ndarray:
    """Softmax along the last axis, shifted by the row maximum."""
    m = np.max(z, axis=-1, keepdims=True)
    e = np.exp(z - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def top_p_select(prob: np.ndarray, top_p: float, valid=None):
    """Top-p selection on rows of block probabilities.

    Returns (order, cum, row_cnt) where order[..., r] is the r-th ranked key
    block (P descending, ties by smaller index), cum[..., r] the inclusive
    cumulative probability of the first r+1 ranked blocks, and row_cnt the
    number of selected blocks k_i.  `valid` (broadcastable to the row shape,
    default nb) is the number of eligible blocks of each row; the others have
    P = 0 and higher indices, so they rank last and are never selected.
    """
    prob = np.asarray(prob, dtype=np.float64)
    nb = prob.shape[-1]
    nvalid = np.broadcast_to(np.int64(nb) if valid is None else np.asarray(valid, dtype=np.int64),
                             prob.shape[:-1])
    order = np.argsort(-prob, axis=-1, kind="stable")
    ranked = np.take_along_axis(prob, order, axis=-1)
    cum = np.cumsum(ranked, axis=-1)
    if top_p >= 1.0:
        row_cnt = nvalid.astype(np.int64).copy()
    else:
        reached = (cum >= top_p) & (np.arange(nb) < nvalid[..., None])
        first = np.argmax(reached, axis=-1) + 1
        row_cnt = np.where(np.any(reached, axis=-1), first, nvalid).astype(np.int64)
    return order, cum, row_cnt


def causal_eligible(nbq: int, nbk: int, block: int, key_block: int) -> np.ndarray:
    """Eligible key blocks per query block under causal routing: key block j
    is eligible for query block i iff j * key_block <= (i+1) * block - 1."""
    last = (np.arange(nbq, dtype=np.int64) + 1) * block - 1
    return np.minimum(nbk, last // key_block + 1)


def causal_cut(scores: np.ndarray, valid=None) -> np.ndarray:
    """Block-level causal cut: Z_ij = -inf for key blocks after the query
    block, j >= valid_i (valid_i = i + 1 when not given: equal block sizes)."""
    nbq, nbk = scores.shape[-2], scores.shape[-1]
    v = np.arange(1, nbq + 1) if valid is None else np.asarray(valid)
    future = np.arange(nbk)[None, :] >= v[:, None]
    return np.where(future, -np.inf, scores)


@dataclasses.dataclass
class RouteResult:
    qbar: np.ndarray        # [B,H,nb,d] float64
    kbar: np.ndarray        # [B,H,nb,d] float64
    scores: np.ndarray      # [B,H,nb,nb] float64
    prob: np.ndarray        # [B,H,nb,nb] float64
    order: np.ndarray       # [B,H,nb,nb] int64, ranked key blocks
    cum: np.ndarray         # [B,H,nb,nb] float64, inclusive cumulative probability
    row_cnt: np.ndarray     # [B,H,nb] int64
    mask: np.ndarray        # [B,H,nb,nb] uint8
    row_idx: np.ndarray     # [B,H,nb,nb] int32, ascending selected indices, -1 after row_cnt
    head_cnt: np.ndarray    # [B,H] int64
    top_p: float
    valid: np.ndarray | None = None   # [B,H,nb] int64, eligible key blocks per row (i+1 if causal, else nb; None = nb)


def route(q: np.ndarray, k: np.ndarray, block: int, top_p: float, scale: float | None = None,
          causal: bool = False, key_block: int | None = None) -> RouteResult:
    """Full top-p routing of one batch. q, k: [B, H, N, d] (any float dtype, upcast to fp64).
    With `causal`, row i only considers the eligible key blocks (module docstring);
    key_block (default: block) is the key block size."""
    kb = block if key_block is None else key_block
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    d = q.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    qbar = pool_blocks(q, block)
    kbar = pool_blocks(k, kb)
    scores = block_scores(qbar, kbar, scale)
    nbq, nb = scores.shape[-2], scores.shape[-1]
    if causal:
        elig = causal_eligible(nbq, nb, block, kb) if kb != block else None
        scores = causal_cut(scores, elig)
        per_row = np.arange(1, nbq + 1, dtype=np.int64) if elig is None else elig
        valid = np.broadcast_to(per_row, scores.shape[:-1]).copy()
    else:
        valid = np.full(scores.shape[:-1], nb, dtype=np.int64)
    prob = softmax_rows(scores)
    order, cum, row_cnt = top_p_select(prob, top_p, valid)
    rank_pos = np.arange(nb)
    selected_ranked = rank_pos[None, None, None, :] < row_cnt[..., None]
    mask = np.zeros(prob.shape, dtype=np.uint8)
    np.put_along_axis(mask, order, selected_ranked.astype(np.uint8), axis=-1)
    row_idx = np.full(prob.shape, -1, dtype=np.int32)
    B, H = prob.shape[:2]
    for b in range(B):
        for h in range(H):
            for i in range(nbq):
                sel = np.nonzero(mask[b, h, i])[0]
                row_idx[b, h, i, : sel.size] = sel
    head_cnt = row_cnt.sum(axis=-1)
    return RouteResult(qbar, kbar, scores, prob, order, cum, row_cnt, mask, row_idx,
                       head_cnt, float(top_p), valid)


def ambiguous_blocks(res: RouteResult, window: float = 1e-5) -> np.ndarray:
    """Blocks whose selection could flip under a perturbation of size `window`.

    A selected block is ambiguous when its probability exceeds the first
    unselected block's by at most `window`, and an unselected block when the
    last selected block's probability exceeds its own by at most `window`
    (the two could swap across the cut).  Any block is ambiguous when the
    cumulative probability just before or at its rank lies within `window`
    of p (the count k_i could shift by one).  With p >= 1 every block is
    selected by rule and none is ambiguous.
    """
    prob, order, cum = res.prob, res.order, res.cum
    shape = prob.shape
    nb = shape[-1]
    if res.top_p >= 1.0:
        return np.zeros(shape, dtype=bool)
    k = np.asarray(res.row_cnt)
    valid = np.full(k.shape, nb, dtype=np.int64) if res.valid is None else np.asarray(res.valid)
    ranked = np.take_along_axis(prob, order, axis=-1)
    last_in = np.take_along_axis(ranked, (k - 1)[..., None], axis=-1)
    first_out = np.take_along_axis(ranked, np.minimum(k, nb - 1)[..., None], axis=-1)
    first_out = np.where((k < valid)[..., None], first_out, -np.inf)
    excl = cum - ranked
    near_cut_ranked = (np.abs(excl - res.top_p) <= window) | (np.abs(cum - res.top_p) <= window)
    near_cut = np.zeros(shape, dtype=bool)
    np.put_along_axis(near_cut, order, near_cut_ranked, axis=-1)
    rank_of = np.empty_like(order)
    np.put_along_axis(rank_of, order, np.broadcast_to(np.arange(nb), shape), axis=-1)
    selected = rank_of < k[..., None]
    eligible = np.arange(nb) < valid[..., None]
    swap_in = selected & (prob - first_out <= window)
    swap_out = ~selected & eligible & (last_in - prob <= window)
    return (near_cut & eligible) | swap_in | swap_out
