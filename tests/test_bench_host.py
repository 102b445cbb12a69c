"""Host-side logic of the benchmark: its executed-FLOP count must equal the
oracle's definition (allowed token pairs of the selected block pairs)."""
import numpy as np
import pytest

import bench
import oracle


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,block", [(1000, 64), (1300, 128), (64, 64), (5, 64)])
def test_bench_flops_equal_oracle(N, block, causal):
    rng = np.random.default_rng(N + block)
    nb = oracle.num_blocks(N, block)
    mask = (rng.random((2, 3, nb, nb)) < 0.4).astype(np.uint8)
    if causal:
        mask = mask * np.tril(np.ones((nb, nb), dtype=np.uint8))
    want = sum(oracle.executed_flops(mask[b, h], N, block, 128, causal) for b in range(2) for h in range(3))
    assert bench.executed_flops(mask, N, block, 128, causal) == want
