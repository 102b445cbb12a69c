"""GPU parity of the ranked tail the router leaves after the selected blocks,
of the LPT model for any worker count, and of slack-aware augmentation
priced in row-tiles (attn_augment: the batched assignment, the pairs each
worker buys, the rewritten rows) against the fp64 oracle on the same
routing.  Every call goes through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import top_block_sparse_pool_amd as tbs
from parity import compare_units, to64
from workloads import WORKLOADS, custom_workload, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(w, seed=0):
    print(f"[case] {w.describe()} seed={seed}", flush=True)
    return [t.to(DEV) for t in make_inputs(w, seed)]


def _oracle_route(q, k, block, p, causal):
    return oracle.route(to64(q), to64(k), block, p, causal=causal)


TAIL = [
    (custom_workload(1, 3, 1000, 128, 64, "bf16", 0.8, wid=501), False),
    (custom_workload(1, 2, 1300, 128, 128, "bf16", 0.7, wid=502), True),
    (custom_workload(1, 2, 600, 64, 64, "f32", 0.5, wid=503), False),
]


@pytest.mark.parametrize("w,causal", TAIL, ids=lambda x: getattr(x, "name", str(x)))
def test_route_ranked_tail(w, causal):
    q, k, v = _inputs(w)
    r = tbs.route(q, k, w.top_p, w.block, causal=causal, return_prob=True)
    torch.cuda.synchronize()
    ref = _oracle_route(q, k, w.block, w.top_p, causal)
    prob = r.block_prob.cpu().numpy()
    assert np.abs(prob - ref.prob).max() <= 1e-12
    mask, rc, ri = r.mask.cpu().numpy(), r.row_cnt.cpu().numpy(), r.row_idx.cpu().numpy()
    B, H, nb = rc.shape
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                nv = i + 1 if causal else nb
                kk = int(rc[b, h, i])
                tail = ri[b, h, i, kk:nv]
                assert sorted(tail.tolist()) == np.nonzero(mask[b, h, i, :nv] == 0)[0].tolist()
                pt = prob[b, h, i, tail]
                # ranked: P descending, equal P by smaller index
                assert all(pt[x] > pt[x + 1] or (pt[x] == pt[x + 1] and tail[x] < tail[x + 1])
                           for x in range(len(tail) - 1))


@pytest.mark.parametrize("W", [7, 64, 65, 256, 300, 1024, 4096])
def test_lpt_any_worker_count(W):
    w = custom_workload(2, 5, 2000, 128, 64, "bf16", 0.9, wid=510)
    q, k, v = _inputs(w)
    pr = tbs.make_problem(q, w.block)
    ws = tbs.workspace(pr, DEV)
    r = tbs.route(q, k, w.top_p, w.block, ws=ws)
    wl, worker_of, worker_load = tbs.schedule(pr, r.row_cnt, ws, head_window=2, num_workers=W, lpt=True)
    torch.cuda.synchronize()
    costs = oracle.group_costs(r.row_cnt.cpu().numpy(), pr.group)
    want_of, want_load = oracle.lpt_assign(costs, wl.cpu().numpy(), W)
    assert (worker_of.cpu().numpy() == want_of).all()
    assert (worker_load.cpu().numpy() == want_load).all()


def _rank_order(prob):
    """Every row's key blocks by (P desc, j asc): the router's rank order."""
    nbk = prob.shape[-1]
    j = np.broadcast_to(np.arange(nbk), prob.shape)
    return np.lexsort((j, -prob), axis=-1)


def _valid(pr, causal):
    if not causal:
        return None
    elig = oracle.causal_eligible(pr.num_blocks, pr.num_key_blocks, pr.block, pr.kblock)
    return np.broadcast_to(elig, (pr.batch, pr.heads, pr.num_blocks)).astype(np.int64)


def _augment_and_reference(q, k, w, causal, W, kb=None, hw=2):
    """attn_augment on the GPU's routing, and the oracle on the same routing
    (the GPU's block probabilities, selection and work list).  The problem
    carries FLAG_NO_SPLIT: small problems would otherwise run their forward
    in equal shares, and attn_augment would leave them unchanged."""
    pr = tbs.make_problem(q, w.block, causal=causal, key_block=kb, flags=tbs.FLAG_NO_SPLIT)
    ws = tbs.workspace(pr, DEV)
    r = tbs.route(q, k, w.top_p, w.block, ws=ws, causal=causal, return_prob=True, key_block=kb)
    wl = tbs.schedule(pr, r.row_cnt, ws, head_window=hw)
    torch.cuda.synchronize()
    prob, mask0 = r.block_prob.cpu().numpy(), r.mask.cpu().numpy()
    wl_np = wl.cpu().numpy()
    # the work list is the oracle's (pinned by the scheduler tests): checked again here
    ng = -(-pr.num_blocks // pr.group)
    assert (wl_np == oracle.work_list(oracle.group_costs(r.row_cnt.cpu().numpy(), pr.group), hw * ng)).all()
    aug = tbs.augment(pr, r, ws, work_list=wl, num_workers=W)
    torch.cuda.synchronize()
    ref = oracle.augment(prob, mask0, _rank_order(prob), wl_np, _valid(pr, causal), pr.group, W, w.seq_len,
                         pr.kblock, tbs.SASA_TILE_FIXED)
    return pr, ws, r, wl, aug, ref, prob, mask0


def _check_equal(r, aug, ref):
    assert (aug.worker_of.cpu().numpy() == ref.worker_of).all()
    assert (aug.worker_load.cpu().numpy() == ref.load).all()
    assert (aug.paid.cpu().numpy() == ref.paid).all()
    assert (r.mask.cpu().numpy() == ref.mask).all()
    assert (r.row_cnt.cpu().numpy() == ref.row_cnt).all()
    assert (r.head_cnt.cpu().numpy() == ref.head_cnt).all()
    ri = r.row_idx.cpu().numpy()
    written = ref.row_idx >= 0            # selection and ranked tail; entries after them are not written
    assert (ri[written] == ref.row_idx[written]).all()


AUG = [
    (custom_workload(1, 4, 2000, 128, 64, "bf16", 0.8, wid=520), False, 16, None),     # G = 4
    (custom_workload(1, 4, 2000, 128, 64, "bf16", 0.8, wid=520), False, 256, None),    # W > items
    (custom_workload(1, 4, 2000, 128, 64, "bf16", 0.5, wid=520), False, 1, None),      # one worker: no slack
    (custom_workload(2, 3, 1500, 128, 128, "bf16", 0.7, wid=521), False, 7, None),     # G = 2
    (custom_workload(1, 3, 1000, 128, 128, "bf16", 0.6, wid=525), False, 5, 128),      # ragged 128-key blocks
    (custom_workload(1, 4, 1500, 128, 128, "bf16", 0.6, wid=526), False, 9, 64),       # 128-row blocks over 64 keys
    (custom_workload(1, 3, 900, 64, 64, "f32", 0.6, wid=522), False, 5, None),         # G = 1
    (custom_workload(1, 4, 2000, 128, 64, "bf16", 0.8, wid=523), True, 16, None),      # causal
    (custom_workload(1, 3, 1300, 128, 128, "bf16", 0.7, wid=527), True, 6, 64),        # causal, mixed blocks
    (custom_workload(1, 12, 16384, 64, 64, "bf16", 0.5, wid=524), False, 5, None),     # long lists, few workers
]


@pytest.mark.parametrize("w,causal,W,kb", AUG, ids=lambda x: getattr(x, "name", str(x)))
def test_augment_matches_oracle(w, causal, W, kb):
    q, k, v = _inputs(w)
    pr, ws, r, wl, aug, ref, prob, mask0 = _augment_and_reference(q, k, w, causal, W, kb)
    print(f"  {int(ref.paid.sum())} pairs bought by {W} workers for {int(ref.paid_cost.sum())} row-tiles "
          f"(slack {int(ref.slack.sum())})", flush=True)
    _check_equal(r, aug, ref)
    assert (oracle.retained_mass(prob, ref.mask) >= oracle.retained_mass(prob, mask0)).all()
    # attention over the augmented lists, on the same work list
    o, lse = tbs.sparse_fwd(q, k, v, r.row_cnt, r.row_idx, w.block, work_list=wl, ws=ws, causal=causal,
                            key_block=kb, flags=tbs.FLAG_NO_SPLIT)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    units = [(b, h, int(i)) for b in range(pr.batch) for h in range(pr.heads)
             for i in rng.choice(pr.num_blocks, size=min(3, pr.num_blocks), replace=False)]
    e, le = compare_units(o, lse, q, k, v, w.block, units, ref.mask, q.dtype, causal=causal, key_block=kb)
    print(f"  attention on augmented lists: max |O err| {e:.3e}, |LSE err| {le:.3e}", flush=True)


@pytest.mark.parametrize("W", [7, 64, 65, 300, 1024, 4096])
def test_augment_any_worker_count(W):
    w = custom_workload(2, 5, 2000, 128, 64, "bf16", 0.6, wid=511)
    q, k, v = _inputs(w)
    pr, ws, r, wl, aug, ref, prob, mask0 = _augment_and_reference(q, k, w, False, W)
    _check_equal(r, aug, ref)
    # the assignment is the batched longest-first one over the item costs
    cost = oracle.item_costs(mask0, pr.group, w.seq_len, pr.kblock, tbs.SASA_TILE_FIXED)
    wo, load, last = oracle.lpt_batched(cost, wl.cpu().numpy(), W)
    assert (aug.worker_of.cpu().numpy() == wo).all() and (aug.worker_load.cpu().numpy() == load).all()


def test_augment_full_size_video():
    w = WORKLOADS["video-32k"]
    q, k, v = _inputs(w)
    W = torch.cuda.get_device_properties(0).multi_processor_count
    pr, ws, r, wl, aug, ref, prob, mask0 = _augment_and_reference(q, k, w, False, W,
                                                                   hw=tbs.default_head_window(
                                                                       tbs.make_problem(q, w.block)))
    _check_equal(r, aug, ref)
    m0 = oracle.retained_mass(prob, mask0).mean()
    m1 = oracle.retained_mass(prob, ref.mask).mean()
    print(f"  {W} workers: {int(ref.paid.sum())} pairs bought for {int(ref.paid_cost.sum())} row-tiles, makespan "
          f"{ref.makespan}, mean retained mass {m0:.5f} -> {m1:.5f}", flush=True)
    assert m1 > m0


def test_sparse_attention_with_sasa_end_to_end():
    # 1024 work items: the forward does not split them, so the assignment
    # model describes it and the slack is spent
    w = custom_workload(1, 8, 32768, 128, 64, "bf16", 0.9, wid=530)
    q, k, v = _inputs(w)
    pr = tbs.make_problem(q, w.block)
    ws = tbs.workspace(pr, DEV)
    r0 = tbs.route(q, k, w.top_p, w.block, ws=ws, return_prob=True)
    wl0 = tbs.schedule(pr, r0.row_cnt, ws)
    torch.cuda.synchronize()
    prob, mask0, wl_np = r0.block_prob.cpu().numpy(), r0.mask.cpu().numpy(), wl0.cpu().numpy()
    o, lse, r, wl = tbs.sparse_attention(q, k, v, w.top_p, w.block, sasa=True)
    torch.cuda.synchronize()
    assert (wl.cpu().numpy() == wl_np).all()          # the forward ran on the augmentation's list
    W = tbs.num_workers(pr, tbs.OP_SPARSE_FWD)
    ref = oracle.augment(prob, mask0, _rank_order(prob), wl_np, None, pr.group, W, w.seq_len, pr.kblock,
                         tbs.SASA_TILE_FIXED)
    assert ref.paid.sum() > 0
    assert (r.mask.cpu().numpy() == ref.mask).all()
    mass0 = oracle.retained_mass(prob, mask0).mean()
    mass1 = oracle.retained_mass(prob, ref.mask).mean()
    print(f"  mean retained mass {mass0:.5f} -> {mass1:.5f}, {int(ref.paid.sum())} pairs bought", flush=True)
    rng = np.random.default_rng(3)
    units = [(0, h, int(i)) for h in range(w.heads) for i in rng.choice(pr.num_blocks, size=2, replace=False)]
    compare_units(o, lse, q, k, v, w.block, units, ref.mask, q.dtype)


def test_augment_leaves_split_problems_unchanged():
    # 32 work items: the forward runs them in equal shares of their tiles, so
    # attn_augment buys nothing (and still reports the assignment)
    w = custom_workload(1, 4, 2000, 128, 64, "bf16", 0.6, wid=531)
    q, k, v = _inputs(w)
    pr = tbs.make_problem(q, w.block)
    ws = tbs.workspace(pr, DEV)
    r = tbs.route(q, k, w.top_p, w.block, ws=ws, return_prob=True)
    wl = tbs.schedule(pr, r.row_cnt, ws)
    torch.cuda.synchronize()
    mask0, idx0, cnt0 = r.mask.clone(), r.row_idx.clone(), r.row_cnt.clone()
    aug = tbs.augment(pr, r, ws, work_list=wl, num_workers=16)
    torch.cuda.synchronize()
    assert (aug.paid == 0).all()
    assert torch.equal(r.mask, mask0) and torch.equal(r.row_idx, idx0) and torch.equal(r.row_cnt, cnt0)
    cost = oracle.item_costs(mask0.cpu().numpy(), pr.group, w.seq_len, pr.kblock, tbs.SASA_TILE_FIXED)
    wo, load, _ = oracle.lpt_batched(cost, wl.cpu().numpy(), 16)
    assert (aug.worker_of.cpu().numpy() == wo).all() and (aug.worker_load.cpu().numpy() == load).all()


UNION = [
    (custom_workload(1, 4, 2000, 128, 64, "bf16", 0.8, wid=540), False, None),   # G = 4
    (custom_workload(2, 3, 1500, 128, 128, "bf16", 0.7, wid=541), False, None),  # G = 2
    (custom_workload(1, 4, 2000, 128, 64, "bf16", 0.8, wid=542), True, None),    # causal
    (custom_workload(1, 3, 1000, 128, 128, "bf16", 0.8, wid=543), True, 64),     # causal, key blocks of 64
    (custom_workload(1, 2, 600, 64, 64, "f32", 0.7, wid=544), False, None),      # G = 1: nothing changes
]


@pytest.mark.parametrize("w,causal,kb", UNION, ids=lambda x: getattr(x, "name", str(x)))
def test_augment_union_matches_oracle(w, causal, kb):
    q, k, v = _inputs(w)
    pr = tbs.make_problem(q, w.block, causal=causal, key_block=kb)
    ws = tbs.workspace(pr, DEV)
    r = tbs.route(q, k, w.top_p, w.block, ws=ws, causal=causal, key_block=kb)
    mask0 = r.mask.cpu().numpy()
    tbs.augment_union(pr, r)
    wl = tbs.schedule(pr, r.row_cnt, ws)
    o, lse = tbs.sparse_fwd(q, k, v, r.row_cnt, r.row_idx, w.block, work_list=wl, ws=ws, causal=causal,
                            key_block=kb)
    torch.cuda.synchronize()
    rr = oracle.route(to64(q), to64(k), w.block, w.top_p, causal=causal, key_block=kb)
    assert (mask0 == rr.mask).all(), "routing differs on an ambiguous block; exact comparison not possible"
    ref = oracle.union_fill(rr.mask, rr.order, rr.valid, pr.group)
    assert (r.mask.cpu().numpy() == ref.mask).all()
    assert (r.row_cnt.cpu().numpy() == ref.row_cnt).all()
    assert (r.head_cnt.cpu().numpy() == ref.head_cnt).all()
    ri = r.row_idx.cpu().numpy()
    written = ref.row_idx >= 0                     # selection and ranked tail; entries after them are not written
    assert (ri[written] == ref.row_idx[written]).all()
    print(f"  {int(ref.added.sum())} blocks added to {int(rr.mask.sum())}", flush=True)
    rng = np.random.default_rng(2)
    units = [(b, h, int(i)) for b in range(pr.batch) for h in range(pr.heads)
             for i in rng.choice(pr.num_blocks, size=min(3, pr.num_blocks), replace=False)]
    compare_units(o, lse, q, k, v, w.block, units, ref.mask, q.dtype, causal=causal, key_block=kb)
