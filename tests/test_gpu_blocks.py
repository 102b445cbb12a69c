"""GPU parity with query and key blocks of different sizes (block != key_block)
against the fp64 oracle: routing over key blocks of their own size, the
causal eligibility of key blocks, attention over the listed key blocks, and
p = 1 equal to dense attention bit for bit.  Every call goes through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import top_block_sparse_pool_amd as tbs
from parity import compare_route, compare_units, oracle_route_per_head, routed_units, to64
from workloads import WORKLOADS, custom_workload, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(w, seed=0):
    print(f"[case] {w.describe()} seed={seed}", flush=True)
    return [t.to(DEV) for t in make_inputs(w, seed)]


CASES = [
    (custom_workload(1, 3, 1000, 128, 128, "bf16", 0.9, wid=601), 64, False),    # nbq 8, nbk 16, tail 40
    (custom_workload(1, 3, 1000, 128, 128, "bf16", 0.8, wid=601), 64, True),
    (custom_workload(2, 2, 1500, 128, 64, "bf16", 0.9, wid=602), 128, False),    # nbq 24, nbk 12, tail 92
    (custom_workload(2, 2, 1500, 128, 64, "bf16", 0.7, wid=602), 128, True),
    (custom_workload(1, 2, 777, 64, 128, "bf16", 0.9, wid=603), 64, True),       # d = 64
    (custom_workload(1, 2, 700, 64, 64, "f32", 0.8, wid=604), 128, False),       # fp32
    (custom_workload(1, 2, 600, 128, 128, "f32", 0.8, wid=605), 64, True),
    (custom_workload(1, 1, 5, 128, 128, "bf16", 0.9, wid=606), 64, False),       # N < both blocks
]


@pytest.mark.parametrize("w,kb,causal", CASES, ids=lambda x: getattr(x, "name", str(x)))
def test_mixed_blocks_path_matches_oracle(w, kb, causal):
    q, k, v = _inputs(w)
    pr = tbs.make_problem(q, w.block, causal=causal, key_block=kb)
    ws = tbs.workspace(pr, DEV)
    r = tbs.route(q, k, w.top_p, w.block, ws=ws, causal=causal, key_block=kb, return_prob=True)
    wl = tbs.schedule(pr, r.row_cnt, ws)
    o, lse = tbs.sparse_fwd(q, k, v, r.row_cnt, r.row_idx, w.block, work_list=wl, ws=ws, causal=causal,
                            key_block=kb)
    torch.cuda.synchronize()
    nb, nbk = pr.num_blocks, pr.num_key_blocks
    assert r.mask.shape == (pr.batch, pr.heads, nb, nbk)
    ref = oracle_route_per_head(q, k, w.block, w.top_p, causal=causal, key_block=kb)
    cmp = compare_route(r, ref)
    if causal:
        e = oracle.causal_eligible(nb, nbk, w.block, kb)
        assert not (r.mask.cpu().numpy() * (np.arange(nbk)[None, :] >= e[:, None])).any()
    G = pr.group
    want_wl = oracle.work_list(oracle.group_costs(r.row_cnt.cpu().numpy(), G),
                               tbs.default_head_window(pr) * -(-nb // G))
    assert (wl.cpu().numpy() == want_wl).all()
    units = [(b, h, i) for b in range(pr.batch) for h in range(pr.heads) for i in range(nb)]
    err, lerr = compare_units(o, lse, q, k, v, w.block, units, cmp["gpu_mask"], q.dtype, causal=causal,
                              key_block=kb)
    print(f"  {len(units)} blocks: max |O err| {err:.3e}, |LSE err| {lerr:.3e}", flush=True)


@pytest.mark.parametrize("w,kb,causal", [CASES[0], CASES[1], CASES[2], CASES[5], CASES[6]],
                         ids=lambda x: getattr(x, "name", str(x)))
def test_mixed_blocks_p1_equals_dense_bitwise(w, kb, causal):
    q, k, v = _inputs(w, seed=1)
    pr = tbs.make_problem(q, w.block, causal=causal, key_block=kb)
    ws = tbs.workspace(pr, DEV)
    r = tbs.route(q, k, 1.0, w.block, ws=ws, causal=causal, key_block=kb)
    ns = tbs.FLAG_NO_SPLIT   # both calls run every work item whole
    o, lse = tbs.sparse_fwd(q, k, v, r.row_cnt, r.row_idx, w.block, ws=ws, causal=causal, key_block=kb, flags=ns)
    od, lsed = tbs.dense_fwd(q, k, v, w.block, causal=causal, ws=ws, flags=ns)
    torch.cuda.synchronize()
    nb, nbk = pr.num_blocks, pr.num_key_blocks
    want = np.ones((nb, nbk), dtype=np.uint8)
    if causal:
        want = (np.arange(nbk)[None, :] < oracle.causal_eligible(nb, nbk, w.block, kb)[:, None]).astype(np.uint8)
    assert (r.mask.cpu().numpy() == want[None, None]).all()
    assert torch.equal(o, od) and torch.equal(lse, lsed)


def test_mixed_blocks_full_size_video_sample():
    # The video shape routed with 128-row query blocks over 64-key blocks.
    w = WORKLOADS["video-32k"]
    q, k, v = _inputs(w)
    bq, kb = 128, 64
    pr = tbs.make_problem(q, bq, key_block=kb)
    ws = tbs.workspace(pr, DEV)
    r = tbs.route(q, k, w.top_p, bq, ws=ws, key_block=kb)
    wl = tbs.schedule(pr, r.row_cnt, ws)
    o, lse = tbs.sparse_fwd(q, k, v, r.row_cnt, r.row_idx, bq, work_list=wl, ws=ws, key_block=kb)
    torch.cuda.synchronize()
    print("  gpu done; oracle routing", flush=True)
    ref = oracle_route_per_head(q, k, bq, w.top_p, key_block=kb)
    cmp = compare_route(r, ref)
    rc = r.row_cnt.cpu().numpy()
    print(f"  mask ok (ambiguous mismatches {cmp['ambiguous_mismatches']}), density "
          f"{rc.sum() / (pr.units * pr.num_key_blocks):.3f}", flush=True)
    rng = np.random.default_rng(7)
    units = []
    for h in range(0, w.heads, 3):
        cand = {0, pr.num_blocks - 1, int(np.argmax(rc[0, h])), int(rng.integers(pr.num_blocks))}
        units += [(0, h, i) for i in sorted(cand)]
    units = routed_units(units, cmp)
    e, le = compare_units(o, lse, q, k, v, bq, units, cmp["gpu_mask"], q.dtype, key_block=kb)
    print(f"  {len(units)} sampled blocks: max |O err| {e:.3e}, |LSE err| {le:.3e}", flush=True)
