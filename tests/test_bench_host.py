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
