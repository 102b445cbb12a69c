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


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,bq,bk", [(1000, 128, 64), (1300, 64, 128), (5, 128, 64)])
def test_bench_flops_mixed_blocks_equal_oracle(N, bq, bk, causal):
    rng = np.random.default_rng(N + bq)
    nbq, nbk = oracle.num_blocks(N, bq), oracle.num_blocks(N, bk)
    mask = (rng.random((1, 2, nbq, nbk)) < 0.4).astype(np.uint8)
    want = sum(oracle.executed_flops(mask[0, h], N, bq, 64, causal, key_block=bk) for h in range(2))
    assert bench.executed_flops(mask, N, bq, 64, causal, bk) == want


def test_fp8_peak_is_the_harmonic_mix():
    # Half of the FLOPs at the fp8 rate and half at the bf16 rate take
    # 0.5/5.0 + 0.5/2.5 = 0.3 ms per PFLOP, so the peak is 1/0.3 PFLOP/s.
    assert abs(bench.FP8_QK_PEAK_TFLOPS - 1e3 / 0.3) < 1e-6
    assert bench.BF16_PEAK_TFLOPS < bench.FP8_QK_PEAK_TFLOPS < bench.FP8_PEAK_TFLOPS


@pytest.mark.parametrize("heads,gpus", [(40, 8), (24, 8), (40, 3), (7, 7), (5, 8)])
def test_head_split_equals_oracle_lpt(heads, gpus):
    # Whole heads go to GPUs longest first; the oracle's greedy LPT over the
    # stable (cost desc, id asc) order, ties to the lowest worker, is the same rule.
    rng = np.random.default_rng(heads * 31 + gpus)
    costs = rng.integers(1, 60, size=heads) * 512
    costs[:3] = costs[0]                      # ties between heads
    gpu_of, load = bench.head_lpt(costs, gpus)
    want_of, want_load = oracle.lpt_assign(costs, oracle.work_list(costs), gpus)
    assert np.array_equal(gpu_of, want_of)
    assert np.array_equal(load, want_load)
    assert load.sum() == costs.sum()
    assert np.array_equal(bench.contiguous_head_loads(costs, gpus), oracle.static_partition_loads(costs, gpus))


def test_head_split_hand_example():
    # Costs 9 7 5 4 3 over two GPUs: 9 -> g0, 7 -> g1, 5 -> g1 (7 < 9), 4 -> g0 (9 < 12),
    # 3 -> g1 (12 < 13).  Contiguous halves: heads 0-1 (16) and 2-4 (12).
    gpu_of, load = bench.head_lpt([9, 7, 5, 4, 3], 2)
    assert gpu_of.tolist() == [0, 1, 1, 0, 1]
    assert load.tolist() == [13, 15]
    assert bench.contiguous_head_loads([9, 7, 5, 4, 3], 2).tolist() == [16, 12]
