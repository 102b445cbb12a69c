"""Host-side logic of the benchmark: its executed-FLOP count must equal the
oracle's definition (allowed token pairs of the selected block pairs)."""
import os

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


def test_metric_names_the_shape_run():
    # The headline string is the one built for the 32k video shape; a head
    # share or another workload names its own shape.
    assert bench.metric_for(32760, 40, 128, "bf16") == bench.METRIC
    assert "H=5 " in bench.metric_for(32760, 5, 128, "bf16")
    assert "N=118800 H=24" in bench.metric_for(118800, 24, 128, "bf16")
    assert "causal" in bench.metric_for(32760, 40, 128, "bf16", causal=True)


def test_union_tiles_counts_item_unions():
    # 5 query blocks of 64 over 3 key blocks of 128 (last one 40 keys: 1 tile),
    # items of 2 query blocks: {0,1}, {2,3}, {4}.
    mask = np.array([[1, 0, 0],
                     [0, 1, 0],
                     [1, 0, 1],
                     [1, 0, 0],
                     [0, 0, 1]], dtype=np.uint8)[None, None]
    N = 2 * 128 + 40
    # item 0: blocks 0,1 -> 2 + 2 tiles; item 1: blocks 0,2 -> 2 + 1; item 2: block 2 -> 1
    assert bench.union_tiles(mask, N, 64, 128, 2) == 8
    # one block per item: the per-row sum
    assert bench.union_tiles(mask, N, 64, 128, 1) == 2 + 2 + 3 + 2 + 1


def test_summarize_counters_scales_by_the_copy(tmp_path):
    import sqlite3

    def db(path, counter, copy_kib, kernel_kib):
        con = sqlite3.connect(path)
        con.execute("create table counters_collection (dispatch_id int, kernel_name text, counter_name text, "
                    "value real)")
        rows = [(1, "__amd_rocclr_copyBuffer", counter, copy_kib)]
        rows += [(2 + i, "void ns::flash_fwd_bf16_pp<128, 64, 64, 0, false>(P)", counter, v)
                 for i, v in enumerate(kernel_kib)]
        rows += [(9, "void ns::other(P)", counter, 5.0)]
        con.executemany("insert into counters_collection values (?, ?, ?, ?)", rows)
        con.commit()
        con.close()
        return str(path)

    f = db(tmp_path / "f.db", "FETCH_SIZE", 512 * 1024, [1000.0, 3000.0, 2000.0, 9999.0])
    w = db(tmp_path / "w.db", "WRITE_SIZE", 1024 * 1024, [10.0, 30.0, 20.0, 99.0])
    res = bench.summarize_counters(f, w, "flash_fwd_bf16_pp<128, 64, 64, 0, false>", 1024, 3)
    assert res["fetch_scale"] == 2.0 and res["write_scale"] == 1.0
    assert res["fetch_bytes_per_launch"] == 2000.0 * 1024 * 2.0      # mean of the first three, scaled
    assert res["write_bytes_per_launch"] == 20.0 * 1024


def test_summarize_trace_timed_dispatches(tmp_path):
    import sqlite3
    path = str(tmp_path / "t.db")
    con = sqlite3.connect(path)
    con.execute("create table kernels (name text, start int, duration int)")
    durs = [900, 800, 100, 200, 300, 400, 5000]            # 2 warm-up, 4 timed, then other launches
    con.executemany("insert into kernels values (?, ?, ?)",
                    [("void ns::flash_fwd_bf16_pp<128, 64, 64, 0, false>(P)", i, d * 1000) for i, d in enumerate(durs)]
                    + [("ns::schedule_kernel(int)", 100 + i, 7000) for i in range(3)])
    con.commit()
    con.close()
    res = bench.summarize_trace(path, "flash_fwd_bf16_pp<128, 64, 64, 0, false>", 2, 4)
    assert res["timed_dispatches"] == 4 and res["timed_mean_us"] == 250.0
    assert res["timed_min_us"] == 100.0 and res["timed_max_us"] == 400.0
    names = [r[0] for r in res["table"]]
    assert len(names) == 2 and res["table"][0][1] == 7


def test_unit_lif_hand_example():
    # costs 5, 1, 4, 2 over two workers: static halves [5+1, 4+2] = [6, 6];
    # longest first 5 -> w0, 4 -> w1, 2 -> w1 (4 < 5), 1 -> w0 (5 < 6): [6, 6]
    r = bench.unit_lif([5, 1, 4, 2], 2)
    assert r["units"] == 4 and r["static_partition"] == 1.0 and r["longest_first_lpt"] == 1.0
    # costs 4, 4, 1, 1 over two workers: static [8, 2] -> 8 / 5; LPT [5, 5] -> 1
    r = bench.unit_lif([4, 4, 1, 1], 2)
    assert abs(r["static_partition"] - 1.6) < 1e-12 and r["longest_first_lpt"] == 1.0
    # windows of two units: [4, 4] then [1, 1] -> 4 -> w0, 4 -> w1, 1 -> w0, 1 -> w1: [5, 5]
    r = bench.unit_lif([4, 4, 1, 1], 2, window_units=2)
    assert r["longest_first_lpt_windowed"] == 1.0
    # windows change the order: [1, 9 | 8, 2] over two workers, windows of two:
    # 9 -> w0, 1 -> w1, 8 -> w1, 2 -> w0 (9 = 9, lowest id) = [11, 9] -> 11 / 10;
    # pure: 9, 8, 2, 1 -> [10, 10]
    r = bench.unit_lif([1, 9, 8, 2], 2, window_units=2)
    assert abs(r["longest_first_lpt_windowed"] - 1.1) < 1e-12 and r["longest_first_lpt"] == 1.0


def test_committed_traffic_summaries_match_their_keys():
    # Each committed HBM counter summary names the workload it is read for; a
    # summary filed under the wrong key would silently drop the traffic field
    # (a summary taken on older kernel sources drops it on purpose).
    import re
    for key, rel in bench.TRAFFIC_SUMMARIES.items():
        with open(os.path.join(bench.ROOT, rel)) as f:
            fields = dict(re.findall(r"^- (\w+): (\S+)\s*$", f.read(), flags=re.M))
        assert fields["workload"] == key, rel
        assert len(fields["kernel_source_sha256"]) == 64, rel
        assert float(fields["fetch_bytes_per_launch"]) > 0 and float(fields["write_bytes_per_launch"]) > 0, rel


def test_summarize_pmc_means_and_clock(tmp_path):
    import sqlite3
    path = str(tmp_path / "p.db")
    con = sqlite3.connect(path)
    con.execute("create table counters_collection (dispatch_id int, kernel_name text, counter_name text, "
                "value real, duration int)")
    k = "void ns::flash_fwd_bf16_pp<128, 64, 64, 0, false>(P)"
    rows = []
    # two dispatches of 1 ms and 2 ms; GRBM_GUI_ACTIVE summed over 8 XCDs at 2 GHz and 1.5 GHz,
    # stored as two rows per dispatch (the halves add up)
    for disp, dur, ghz in ((1, 1_000_000, 2.0), (2, 2_000_000, 1.5)):
        total = ghz * dur * 8
        rows += [(disp, k, "GRBM_GUI_ACTIVE", total / 2, dur), (disp, k, "GRBM_GUI_ACTIVE", total / 2, dur)]
        rows += [(disp, k, "MfmaUtil", 50.0 + disp, dur)]
    rows += [(3, "ns::other(int)", "MfmaUtil", 0.0, 1000)]
    con.executemany("insert into counters_collection values (?, ?, ?, ?, ?)", rows)
    con.commit()
    con.close()
    out = {name: (n, ms, m) for name, n, ms, m in bench.summarize_pmc(path)}
    n, ms, m = out[k]
    assert n == 2 and ms == 1.5
    assert m["MfmaUtil"] == 51.5
    assert abs(m["clock_ghz"] - 1.75) < 1e-12
    assert abs(m["GRBM_GUI_ACTIVE"] - (2.0 * 1e6 * 8 + 1.5 * 2e6 * 8) / 2) < 1e-6
    assert out["ns::other(int)"][0] == 1


def test_issued_flops_counts_full_blocks():
    # two selected pairs in a ragged 2x2 block grid: issued counts both as full
    # 64x64 blocks, executed only the valid tokens (N = 100: blocks of 64 and 36)
    mask = np.array([[1, 0], [1, 1]], dtype=np.uint8)[None, None]
    assert bench.issued_flops(mask, 64, 128) == 4 * 128 * 64 * 64 * 3
    assert bench.issued_flops(mask, 128, 64, key_block=64) == 4 * 64 * 128 * 64 * 3
    assert bench.executed_flops(mask, 100, 64, 128) == 4 * 128 * (64 * 64 + 36 * 64 + 36 * 36)
