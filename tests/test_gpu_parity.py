"""GPU parity against the fp64 oracle at sizes the oracle finishes in seconds:
several tiles, ragged tails, both dtypes, both head dims, both block sizes,
sparse, dense and causal, plus determinism and edge cases.  Every call goes
through the C ABI (the ctypes binding)."""
import itertools
import sys

import numpy as np
import pytest
import torch

import oracle
import top_block_sparse_pool_amd as tbs
from parity import compare_route, compare_units, oracle_route_per_head, to64
from workloads import WORKLOADS, custom_workload, make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _inputs(w, seed=0):
    print(f"[case] {w.describe()} seed={seed}", flush=True)
    return [t.to(DEV) for t in make_inputs(w, seed)]


def _all_units(B, H, nb):
    return [(b, h, i) for b in range(B) for h in range(H) for i in range(nb)]


def _run_sparse(w, q, k, v):
    pr = tbs.make_problem(q, w.block)
    ws = tbs.workspace(pr, DEV)
    r = tbs.route(q, k, w.top_p, w.block, ws=ws)
    wl, worker_of, worker_load = tbs.schedule(pr, r.row_cnt, ws, head_window=w.heads // 2 or 1, lpt=True)
    o, lse = tbs.sparse_fwd(q, k, v, r.row_cnt, r.row_idx, w.block, work_list=wl, ws=ws)
    torch.cuda.synchronize()
    return pr, ws, r, (wl, worker_of, worker_load), o, lse


SMALL_SPARSE = [
    custom_workload(1, 3, 1000, 128, 64, "bf16", 0.9, wid=201),     # nb 16, tail 40
    custom_workload(2, 2, 1500, 128, 128, "bf16", 0.9, wid=202),    # nb 12, tail 92 (two key tiles)
    custom_workload(1, 2, 1300, 128, 128, "bf16", 0.95, wid=203),   # nb 11, tail 20 (second tile empty)
    custom_workload(1, 4, 700, 64, 64, "bf16", 0.8, wid=204),       # d = 64
    custom_workload(1, 2, 777, 64, 128, "bf16", 0.9, wid=205),      # d = 64, block 128
    custom_workload(1, 2, 600, 128, 64, "f32", 0.9, wid=206),       # fp32, d = 128
    custom_workload(1, 2, 300, 64, 128, "f32", 0.7, wid=207),       # fp32, block 128
    custom_workload(1, 2, 64, 128, 64, "bf16", 0.5, wid=208),       # a single block
    custom_workload(1, 1, 5, 128, 64, "bf16", 0.9, wid=209),        # N < block
]


@pytest.mark.parametrize("w", SMALL_SPARSE, ids=lambda w: w.name)
def test_sparse_path_matches_oracle(w):
    q, k, v = _inputs(w)
    pr, ws, r, (wl, worker_of, worker_load), o, lse = _run_sparse(w, q, k, v)
    ref = oracle_route_per_head(q, k, w.block, w.top_p)
    cmp = compare_route(r, ref)
    print(f"  ambiguous mismatches: {cmp['ambiguous_mismatches']}", flush=True)
    # scheduler: exact work list and LPT model
    G = pr.group
    ng = -(-pr.num_blocks // G)
    costs = oracle.group_costs(r.row_cnt.cpu().numpy(), G)
    want_wl = oracle.work_list(costs, (w.heads // 2 or 1) * ng)
    assert (wl.cpu().numpy() == want_wl).all()
    W = worker_load.numel()
    want_of, want_load = oracle.lpt_assign(costs, want_wl, W)
    assert (worker_of.cpu().numpy() == want_of).all()
    assert (worker_load.cpu().numpy() == want_load).all()
    # attention on every query block, against the oracle on the GPU's own mask
    B, H, nb = pr.batch, pr.heads, pr.num_blocks
    units = _all_units(B, H, nb)
    dt = q.dtype
    e, le = compare_units(o, lse, q, k, v, w.block, units, cmp["gpu_mask"], dt)
    print(f"  max |O err| {e:.3e}  max |LSE err| {le:.3e} over {len(units)} blocks", flush=True)
    # processing order does not change a single bit
    o2, lse2 = tbs.sparse_fwd(q, k, v, r.row_cnt, r.row_idx, w.block, work_list=None, ws=ws)
    o3, lse3 = tbs.sparse_fwd(q, k, v, r.row_cnt, r.row_idx, w.block, work_list=wl, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    assert torch.equal(o, o3) and torch.equal(lse, lse3)


@pytest.mark.parametrize("head_window", [0, 1, 3, 100])
def test_schedule_windows_match_oracle(head_window):
    w = custom_workload(2, 5, 2000, 128, 64, "bf16", 0.9, wid=215)
    q, k, v = _inputs(w)
    pr = tbs.make_problem(q, w.block)
    ws = tbs.workspace(pr, DEV)
    r = tbs.route(q, k, w.top_p, w.block, ws=ws)
    wl, worker_of, worker_load = tbs.schedule(pr, r.row_cnt, ws, head_window=head_window, num_workers=7, lpt=True)
    torch.cuda.synchronize()
    G = pr.group
    costs = oracle.group_costs(r.row_cnt.cpu().numpy(), G)
    want = oracle.work_list(costs, head_window * -(-pr.num_blocks // G))
    assert (wl.cpu().numpy() == want).all()
    want_of, want_load = oracle.lpt_assign(costs, want, 7)
    assert (worker_of.cpu().numpy() == want_of).all() and (worker_load.cpu().numpy() == want_load).all()
    assert (ws[:256] == 0).all()


def test_tiny_fp32_workload_and_p1_equals_dense():
    w = WORKLOADS["tiny-fp32"]
    q, k, v = _inputs(w)
    for p in (0.9, 1.0):
        pr = tbs.make_problem(q, w.block)
        ws = tbs.workspace(pr, DEV)
        r = tbs.route(q, k, p, w.block, ws=ws)
        wl = tbs.schedule(pr, r.row_cnt, ws)
        o, lse = tbs.sparse_fwd(q, k, v, r.row_cnt, r.row_idx, w.block, work_list=wl, ws=ws)
        torch.cuda.synchronize()
        ref = oracle_route_per_head(q, k, w.block, p)
        cmp = compare_route(r, ref)
        compare_units(o, lse, q, k, v, w.block, _all_units(1, 2, 4), cmp["gpu_mask"], torch.float32)
        if p == 1.0:
            assert (r.mask == 1).all()
            od, lsed = tbs.dense_fwd(q, k, v, w.block, ws=ws)
            torch.cuda.synchronize()
            assert torch.equal(o, od) and torch.equal(lse, lsed)


DENSE = [
    (custom_workload(1, 4, 1000, 128, 64, "bf16", 1.0, structured=False, wid=301), False),
    (custom_workload(1, 4, 1000, 128, 64, "bf16", 1.0, structured=False, wid=301), True),
    (custom_workload(1, 2, 1100, 128, 128, "bf16", 1.0, structured=False, wid=302), False),
    (custom_workload(1, 2, 1100, 128, 128, "bf16", 1.0, structured=False, wid=302), True),
    (custom_workload(2, 1, 520, 64, 64, "bf16", 1.0, structured=False, wid=303), True),
    (custom_workload(1, 2, 333, 64, 64, "f32", 1.0, structured=False, wid=304), True),
    (custom_workload(1, 2, 400, 128, 128, "f32", 1.0, structured=False, wid=305), False),
]


@pytest.mark.parametrize("w,causal", DENSE, ids=lambda x: getattr(x, "name", str(x)))
def test_dense_matches_oracle(w, causal):
    q, k, v = _inputs(w)
    o, lse = tbs.dense_fwd(q, k, v, w.block, causal=causal)
    torch.cuda.synchronize()
    nb = -(-w.seq_len // w.block)
    compare_units(o, lse, q, k, v, w.block, _all_units(w.batch, w.heads, nb), None, q.dtype, causal=causal)


@pytest.mark.parametrize("causal", [False, True])
def test_dense_4k_workload(causal):
    w = WORKLOADS["dense-4k"]
    q, k, v = _inputs(w)
    o, lse = tbs.dense_fwd(q, k, v, w.block, causal=causal)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    nb = w.num_blocks
    units = [(0, 0, i) for i in range(nb)] + [(0, int(h), int(rng.integers(nb))) for h in range(1, w.heads)]
    e, le = compare_units(o, lse, q, k, v, w.block, units, None, q.dtype, causal=causal)
    print(f"  dense-4k causal={causal}: max |O err| {e:.3e}, |LSE err| {le:.3e}", flush=True)


def test_sparse_p1_equals_dense_bitwise():
    w = custom_workload(1, 3, 1000, 128, 64, "bf16", 1.0, wid=310)
    q, k, v = _inputs(w)
    pr = tbs.make_problem(q, w.block)
    ws = tbs.workspace(pr, DEV)
    r = tbs.route(q, k, 1.0, w.block, ws=ws)
    wl = tbs.schedule(pr, r.row_cnt, ws)
    ns = tbs.FLAG_NO_SPLIT   # both calls run every work item whole
    o, lse = tbs.sparse_fwd(q, k, v, r.row_cnt, r.row_idx, w.block, work_list=wl, ws=ws, flags=ns)
    od, lsed = tbs.dense_fwd(q, k, v, w.block, ws=ws, flags=ns)
    torch.cuda.synchronize()
    assert (r.mask == 1).all() and (r.row_cnt == r.mask.shape[-1]).all()
    assert torch.equal(o, od) and torch.equal(lse, lsed)


def test_empty_rows_and_hand_made_lists():
    w = custom_workload(1, 2, 300, 128, 64, "bf16", 0.9, wid=320)
    q, k, v = _inputs(w)
    nb = w.num_blocks
    rng = np.random.default_rng(3)
    mask = (rng.random((1, 2, nb, nb)) < 0.5).astype(np.uint8)
    mask[0, 0, 1] = 0                               # an empty row
    mask[0, 1, 2] = 0
    mask[0, 1, 2, nb - 1] = 1                       # only the ragged tail block
    row_cnt = mask.sum(-1).astype(np.int32)
    row_idx = np.zeros((1, 2, nb, nb), dtype=np.int32)
    for h, i in itertools.product(range(2), range(nb)):
        sel = np.nonzero(mask[0, h, i])[0]
        row_idx[0, h, i, :sel.size] = sel
    rc = torch.from_numpy(row_cnt).to(DEV)
    ri = torch.from_numpy(row_idx).to(DEV)
    o, lse = tbs.sparse_fwd(q, k, v, rc, ri, w.block)
    torch.cuda.synchronize()
    assert (o[0, 0, 64:128] == 0).all() and torch.isneginf(lse[0, 0, 64:128]).all()
    units = [(0, h, i) for h in range(2) for i in range(nb) if row_cnt[0, h, i] > 0]
    compare_units(o, lse, q, k, v, w.block, units, mask, q.dtype)


def test_worker_profile_stamps():
    w = custom_workload(1, 4, 2000, 128, 64, "bf16", 0.9, wid=330)
    q, k, v = _inputs(w)
    pr = tbs.make_problem(q, w.block, flags=tbs.FLAG_PROFILE_WORKERS)
    ws = tbs.workspace(pr, DEV)
    r = tbs.route(q, k, w.top_p, w.block, ws=ws)
    wl = tbs.schedule(pr, r.row_cnt, ws)
    tbs.sparse_fwd(q, k, v, r.row_cnt, r.row_idx, w.block, work_list=wl, ws=ws, flags=tbs.FLAG_PROFILE_WORKERS)
    torch.cuda.synchronize()
    W = tbs.num_workers(pr, tbs.OP_SPARSE_FWD)
    stamps = ws[256:256 + 16 * W].view(torch.int64).view(W, 2).cpu()
    assert W >= 1 and (stamps[:, 1] >= stamps[:, 0]).all() and (stamps[:, 0] > 0).all()
    assert (ws[:256] == 0).all()     # queue counters left at zero


def test_one_gpu_share_equals_the_full_problem_on_its_heads():
    # bench.py --share-of G runs the heads that the head-level LPT gives one
    # GPU as a problem of their own; heads are independent and the results do
    # not depend on the processing order, so the share's masks, counts,
    # outputs and LSE equal the full problem's rows of those heads bit for bit
    # when neither call splits its work items along their keys (both are
    # small enough that the default calls do; those agree to rounding).
    import bench
    w = custom_workload(1, 8, 1500, 128, 64, "bf16", 0.9, wid=217)
    q, k, v = _inputs(w)
    pr = tbs.make_problem(q, w.block)
    ws = tbs.workspace(pr, DEV)
    r = tbs.route(q, k, w.top_p, w.block, ws=ws)
    wl = tbs.schedule(pr, r.row_cnt, ws)
    o, lse = tbs.sparse_fwd(q, k, v, r.row_cnt, r.row_idx, w.block, work_list=wl, ws=ws, flags=tbs.FLAG_NO_SPLIT)
    o_sp, lse_sp = tbs.sparse_fwd(q, k, v, r.row_cnt, r.row_idx, w.block, work_list=wl, ws=ws)
    qs, ks, vs, info = bench.take_share(tbs, q, k, v, w.top_p, w.block, w.block, False, 3)
    heads = info["heads"]
    assert 1 <= len(heads) < w.heads and info["lif_head_lpt"] <= info["lif_contiguous_heads"] + 1e-12
    prs = tbs.make_problem(qs, w.block)
    wss = tbs.workspace(prs, DEV)
    rs = tbs.route(qs, ks, w.top_p, w.block, ws=wss)
    wls = tbs.schedule(prs, rs.row_cnt, wss)
    os_, lses = tbs.sparse_fwd(qs, ks, vs, rs.row_cnt, rs.row_idx, w.block, work_list=wls, ws=wss,
                               flags=tbs.FLAG_NO_SPLIT)
    os_sp, lses_sp = tbs.sparse_fwd(qs, ks, vs, rs.row_cnt, rs.row_idx, w.block, work_list=wls, ws=wss)
    torch.cuda.synchronize()
    idx = torch.tensor(heads, device=DEV)
    assert torch.equal(rs.mask[0], r.mask[0].index_select(0, idx))
    assert torch.equal(rs.row_cnt[0], r.row_cnt[0].index_select(0, idx))
    assert torch.equal(os_[0], o[0].index_select(0, idx))
    assert torch.equal(lses[0], lse[0].index_select(0, idx))
    for a, b in ((o_sp, o), (os_sp, os_)):
        assert (a.float() - b.float()).abs().max().item() <= 2e-2
    for a, b in ((lse_sp, lse), (lses_sp, lses)):
        assert (a - b).abs().max().item() <= 2e-3
    assert sorted(info["head_cost"]) == sorted(int(c) for c in r.head_cnt[0].index_select(0, idx).tolist())
