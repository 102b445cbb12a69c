"""GPU edge cases against the fp64 oracle: exact ties in the block scores,
the largest sizes the C ABI accepts (1024 key blocks for routing, 2048 for
the sparse forward), and p so small that every row keeps one block.  Every
call goes through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import top_block_sparse_pool_amd as tbs
from parity import compare_route, compare_units, oracle_route_per_head, to64
from workloads import custom_workload, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(w, seed=0):
    print(f"[case] {w.describe()} seed={seed}", flush=True)
    return [t.to(DEV) for t in make_inputs(w, seed)]


@pytest.mark.parametrize("causal", [False, True])
def test_exact_ties_take_lowest_indices(causal):
    # Q = 0 makes every block score 0: each row's probabilities are exactly
    # equal, and the tie rule (smaller index first) decides the selection.
    w = custom_workload(1, 2, 64 * 512, 128, 64, "bf16", 0.9, wid=701)
    q, k, v = _inputs(w)
    q.zero_()
    r = tbs.route(q, k, w.top_p, w.block, causal=causal, return_prob=True)
    torch.cuda.synchronize()
    ref = oracle_route_per_head(q, k, w.block, w.top_p, causal=causal)
    cmp = compare_route(r, ref)
    print(f"  ambiguous mismatches {cmp['ambiguous_mismatches']}", flush=True)
    mask = r.mask.cpu().numpy()
    if not causal:
        assert (r.row_cnt == 461).all()                      # ceil(0.9 * 512), sums of 1/512 are exact
        want = np.zeros(512, dtype=np.uint8)
        want[:461] = 1
        assert (mask == want).all()
    else:
        for i in (0, 1, 3, 7, 15, 63, 255, 511):              # i+1 a power of two: exact sums
            kk = int(np.ceil(0.9 * (i + 1)))
            assert (mask[:, :, i, :kk] == 1).all() and (mask[:, :, i, kk:] == 0).all()


def test_largest_routing_size():
    # 1024 key blocks per sequence, the router's limit, with a ragged tail.
    w = custom_workload(1, 2, 64 * 1024 - 24, 128, 64, "bf16", 0.9, wid=702)
    q, k, v = _inputs(w)
    pr = tbs.make_problem(q, w.block)
    assert pr.num_key_blocks == 1024
    ws = tbs.workspace(pr, DEV)
    r = tbs.route(q, k, w.top_p, w.block, ws=ws)
    wl = tbs.schedule(pr, r.row_cnt, ws)
    o, lse = tbs.sparse_fwd(q, k, v, r.row_cnt, r.row_idx, w.block, work_list=wl, ws=ws)
    torch.cuda.synchronize()
    ref = oracle_route_per_head(q, k, w.block, w.top_p)
    cmp = compare_route(r, ref)
    assert (wl.cpu().numpy() == oracle.work_list(oracle.group_costs(r.row_cnt.cpu().numpy(), pr.group),
                                                 tbs.default_head_window(pr) * -(-1024 // pr.group))).all()
    units = [(0, h, i) for h in range(2) for i in (0, 511, 1023) if cmp["rows_agree"][0, h, i]]
    e, le = compare_units(o, lse, q, k, v, w.block, units, ref["mask"], q.dtype)
    print(f"  ambiguous mismatches {cmp['ambiguous_mismatches']}; max |O err| {e:.3e}", flush=True)


def test_largest_sparse_forward_size():
    # 2048 key blocks (the forward's limit) with hand-made lists: every row
    # keeps a few random blocks and the ragged last one.
    w = custom_workload(1, 1, 64 * 2048 - 8, 128, 64, "bf16", 0.9, wid=703)
    q, k, v = _inputs(w)
    nb = 2048
    rng = np.random.default_rng(5)
    mask = np.zeros((1, 1, nb, nb), dtype=np.uint8)
    for i in range(nb):
        mask[0, 0, i, rng.choice(nb - 1, size=3, replace=False)] = 1
        mask[0, 0, i, nb - 1] = 1
    row_cnt = mask.sum(-1).astype(np.int32)
    row_idx = np.zeros((1, 1, nb, nb), dtype=np.int32)
    for i in range(nb):
        sel = np.nonzero(mask[0, 0, i])[0]
        row_idx[0, 0, i, :sel.size] = sel
    o, lse = tbs.sparse_fwd(q, k, v, torch.from_numpy(row_cnt).to(DEV), torch.from_numpy(row_idx).to(DEV), w.block)
    torch.cuda.synchronize()
    units = [(0, 0, int(i)) for i in (0, 1, 1000, 2046, 2047)]
    e, le = compare_units(o, lse, q, k, v, w.block, units, mask, q.dtype)
    print(f"  max |O err| {e:.3e}, |LSE err| {le:.3e}", flush=True)


def test_tiny_p_keeps_one_block_per_row():
    w = custom_workload(1, 3, 2000, 128, 64, "bf16", 1e-9, wid=704)
    q, k, v = _inputs(w)
    r = tbs.route(q, k, w.top_p, w.block, return_prob=True)
    torch.cuda.synchronize()
    assert (r.row_cnt == 1).all()
    prob = r.block_prob.cpu().numpy()
    assert (r.row_idx[..., 0].cpu().numpy() == np.argmax(prob, axis=-1)).all()
    compare_route(r, oracle_route_per_head(q, k, w.block, w.top_p))
