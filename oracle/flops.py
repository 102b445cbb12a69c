"""Executed-work accounting for a block mask (oracle; test infrastructure only).

Each selected (query block i, key block j) pair costs two matrix products,
Q_i K_j^T and P_ij V_j, of 2 * n_i * n_j * d flops each (n = valid tokens);
softmax and exponentials are not counted, by the usual convention for
attention kernels.  Dense attention over N tokens is 4 * N^2 * d per head, and
causal attention counts the N(N+1)/2 allowed (query, key) pairs.
"""
from __future__ import annotations

import numpy as np

from .routing import block_sizes


def executed_flops(mask, n_tokens: int, block: int, head_dim: int, causal: bool = False,
                   key_block: int | None = None) -> int:
    """4 * d * sum over selected pairs of the allowed (query, key) pairs (exact integer).

    A pair of query block i and key block j allows n_i * m_j token pairs; with
    `causal`, only the pairs with key position s <= query position t count.
    """
    mask = np.asarray(mask)
    kb = block if key_block is None else key_block
    n = block_sizes(n_tokens, block).astype(np.int64)
    m = block_sizes(n_tokens, kb).astype(np.int64)
    if not causal:
        pair = np.outer(n, m)                 # [nbq, nbk]
    else:
        # sum over t in query block i of #{s in key block j : s <= t}
        pair = np.zeros((n.size, m.size), dtype=np.int64)
        for i in range(n.size):
            t = np.arange(i * block, i * block + n[i], dtype=np.int64)
            for j in range(m.size):
                pair[i, j] = np.clip(t - j * kb + 1, 0, m[j]).sum()
    per_row = (mask.astype(np.int64) * pair).sum()
    return int(4 * head_dim * per_row)


def dense_flops(batch: int, heads: int, n_tokens: int, head_dim: int, causal: bool = False) -> int:
    pairs = n_tokens * (n_tokens + 1) // 2 if causal else n_tokens * n_tokens
    return int(4 * batch * heads * head_dim * pairs)
