"""GPU parity at the full named workload sizes, in the launch configuration the
benchmark times (route -> schedule -> persistent sparse kernel on one stream).
The whole block mask, index lists and work list are compared with the oracle;
attention outputs are compared on a sample of query blocks (the heaviest, the
lightest, the last and random ones in every head, plus every block whose mask
row differs from the oracle's inside the window), which the oracle computes one
by one on the GPU's own mask.  The dense 119k run is checked on a block of
every head and on the first and last blocks."""
import numpy as np
import pytest
import torch

import oracle
import top_block_sparse_pool_amd as tbs
from parity import compare_route, compare_units, oracle_route_per_head, routed_units
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _sample_units(row_cnt, per_head_random=1, seed=0):
    rng = np.random.default_rng(seed)
    B, H, nb = row_cnt.shape
    units = []
    for b in range(B):
        for h in range(H):
            c = row_cnt[b, h]
            cand = {int(np.argmax(c)), int(np.argmin(c)), nb - 1}
            cand |= {int(x) for x in rng.integers(0, nb, size=per_head_random)}
            units += [(b, h, i) for i in sorted(cand)]
    return units


@pytest.mark.parametrize("name", ["video-32k", "skewed-32k", "video-119k"])
def test_full_size_sparse_workload(name):
    w = WORKLOADS[name]
    print(f"[case] {w.describe()}", flush=True)
    q, k, v = [t.to(DEV) for t in make_inputs(w, 0)]
    pr = tbs.make_problem(q, w.block)
    ws = tbs.workspace(pr, DEV)
    r = tbs.route(q, k, w.top_p, w.block, ws=ws)
    wl = tbs.schedule(pr, r.row_cnt, ws)
    o, lse = tbs.sparse_fwd(q, k, v, r.row_cnt, r.row_idx, w.block, work_list=wl, ws=ws)
    torch.cuda.synchronize()
    print("  gpu done; oracle routing", flush=True)
    ref = oracle_route_per_head(q, k, w.block, w.top_p)
    cmp = compare_route(r, ref)
    costs = r.row_cnt.cpu().numpy()
    G = pr.group
    want_wl = oracle.work_list(oracle.group_costs(costs, G), tbs.default_head_window(pr) * -(-pr.num_blocks // G))
    assert (wl.cpu().numpy() == want_wl).all()
    density = costs.sum() / (pr.units * pr.num_blocks)
    print(f"  mask ok (ambiguous mismatches {cmp['ambiguous_mismatches']}), density {density:.3f}", flush=True)
    units = routed_units(_sample_units(costs), cmp)
    n_diff = int((~cmp["rows_agree"]).sum())
    e, le = compare_units(o, lse, q, k, v, w.block, units, cmp["gpu_mask"], q.dtype)
    print(f"  {len(units)} sampled blocks ({n_diff} rows whose mask differs inside the window): "
          f"max |O err| {e:.3e}, |LSE err| {le:.3e}", flush=True)


def test_full_size_long_video_dense():
    w = WORKLOADS["video-119k"]
    print(f"[case] dense {w.describe()}", flush=True)
    q, k, v = [t.to(DEV) for t in make_inputs(w, 0)]
    o, lse = tbs.dense_fwd(q, k, v, w.block)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    # a random block of every head, and the first and last blocks (ragged tail of 16 tokens)
    units = [(0, h, int(rng.integers(0, w.num_blocks))) for h in range(w.heads)]
    units += [(0, 0, 0), (0, w.heads - 1, w.num_blocks - 1)]
    units = sorted(set(units))
    e, le = compare_units(o, lse, q, k, v, w.block, units, None, q.dtype)
    print(f"  {len(units)} sampled blocks: max |O err| {e:.3e}, |LSE err| {le:.3e}", flush=True)
