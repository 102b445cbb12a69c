"""GPU parity of causal routing and causal block-sparse attention against the
fp64 oracle: key blocks j > i are cut before the block softmax, keys after
each query token are masked.  Every call goes through the C ABI."""
import itertools

import numpy as np
import pytest
import torch

import oracle
import top_block_sparse_pool_amd as tbs
from parity import compare_route, compare_units, dense_causal_splits, oracle_route_per_head, routed_units
from workloads import WORKLOADS, custom_workload, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(w, seed=0):
    print(f"[case] causal {w.describe()} seed={seed}", flush=True)
    return [t.to(DEV) for t in make_inputs(w, seed)]


def _causal_path(w, q, k, v, top_p=None, ws=None):
    p = w.top_p if top_p is None else top_p
    pr = tbs.make_problem(q, w.block, causal=True)
    ws = tbs.workspace(pr, DEV) if ws is None else ws
    r = tbs.route(q, k, p, w.block, ws=ws, causal=True, return_prob=True)
    wl = tbs.schedule(pr, r.row_cnt, ws)
    o, lse = tbs.sparse_fwd(q, k, v, r.row_cnt, r.row_idx, w.block, work_list=wl, ws=ws, causal=True)
    torch.cuda.synchronize()
    return pr, ws, r, wl, o, lse


SMALL = [
    custom_workload(1, 3, 1000, 128, 64, "bf16", 0.9, wid=401),     # nb 16, tail 40
    custom_workload(2, 2, 1500, 128, 128, "bf16", 0.8, wid=402),    # two key tiles per block, tail 92
    custom_workload(1, 2, 1300, 128, 128, "bf16", 0.95, wid=403),   # tail 20
    custom_workload(1, 4, 700, 64, 64, "bf16", 0.7, wid=404),       # d = 64
    custom_workload(1, 2, 777, 64, 128, "bf16", 0.9, wid=405),      # d = 64, block 128
    custom_workload(1, 2, 600, 128, 64, "f32", 0.9, wid=406),       # fp32
    custom_workload(1, 2, 300, 64, 128, "f32", 0.6, wid=407),       # fp32, block 128
    custom_workload(1, 2, 64, 128, 64, "bf16", 0.5, wid=408),       # a single block
    custom_workload(1, 1, 5, 128, 64, "bf16", 0.9, wid=409),        # N < block
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_causal_sparse_path_matches_oracle(w):
    q, k, v = _inputs(w)
    pr, ws, r, wl, o, lse = _causal_path(w, q, k, v)
    nb = pr.num_blocks
    mask = r.mask.cpu().numpy()
    assert not (mask * np.triu(np.ones((nb, nb), dtype=np.uint8), 1)).any(), "a block after the query block"
    assert (r.block_prob.cpu().numpy()[..., np.triu(np.ones((nb, nb), dtype=bool), 1)] == 0).all()
    ref = oracle_route_per_head(q, k, w.block, w.top_p, causal=True)
    cmp = compare_route(r, ref)
    print(f"  ambiguous mismatches: {cmp['ambiguous_mismatches']}", flush=True)
    G = pr.group
    want_wl = oracle.work_list(oracle.group_costs(r.row_cnt.cpu().numpy(), G),
                               tbs.default_head_window(pr) * -(-nb // G))
    assert (wl.cpu().numpy() == want_wl).all()
    units = [(b, h, i) for b in range(pr.batch) for h in range(pr.heads) for i in range(nb)]
    e, le = compare_units(o, lse, q, k, v, w.block, units, cmp["gpu_mask"], q.dtype, causal=True)
    print(f"  max |O err| {e:.3e}  max |LSE err| {le:.3e} over {len(units)} blocks", flush=True)
    o2, lse2 = tbs.sparse_fwd(q, k, v, r.row_cnt, r.row_idx, w.block, ws=ws, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


@pytest.mark.parametrize("w", [SMALL[0], SMALL[1], SMALL[4], SMALL[5], SMALL[6]], ids=lambda w: w.name)
def test_causal_p1_is_lower_triangle_and_equals_dense_causal_bitwise(w):
    q, k, v = _inputs(w, seed=1)
    pr, ws, r, wl, o, lse = _causal_path(w, q, k, v, top_p=1.0)
    nb = pr.num_blocks
    tri = torch.tril(torch.ones((nb, nb), dtype=torch.uint8, device=DEV))
    assert (r.mask == tri).all()
    assert (r.row_cnt == torch.arange(1, nb + 1, device=DEV, dtype=torch.int32)).all()
    assert (r.head_cnt == nb * (nb + 1) // 2).all()
    od, lsed = tbs.dense_fwd(q, k, v, w.block, causal=True, ws=ws)
    # with every work item whole, both calls give the same bits
    ns = tbs.FLAG_NO_SPLIT
    o_ns, lse_ns = tbs.sparse_fwd(q, k, v, r.row_cnt, r.row_idx, w.block, ws=ws, causal=True, flags=ns)
    od_ns, lsed_ns = tbs.dense_fwd(q, k, v, w.block, causal=True, ws=ws, flags=ns)
    torch.cuda.synchronize()
    assert torch.equal(o_ns, od_ns) and torch.equal(lse_ns, lsed_ns)
    if not dense_causal_splits(w):
        # the sparse call may split its items: equal to rounding
        assert (od.float() - o.float()).abs().max().item() <= 2e-2
        assert (lsed - lse).abs().max().item() <= 2e-3
    else:
        # The dense call splits the longest items along the keys and merges
        # the parts: equal to rounding, and both against the oracle.
        units = [(b, h, i) for b in range(w.batch) for h in range(w.heads) for i in range(nb)]
        compare_units(od, lsed, q, k, v, w.block, units, None, q.dtype, causal=True)
        assert (od.float() - o.float()).abs().max().item() <= 2e-2
        assert (lsed - lse).abs().max().item() <= 2e-3


@pytest.mark.parametrize("block", [64, 128])
def test_causal_lists_with_future_blocks_contribute_nothing(block):
    # Hand-made lists that name blocks after the query block: under causal
    # attention those blocks hold no allowed key, so the result equals the
    # list without them, and a row left with none gets o = 0, lse = -inf.
    w = custom_workload(1, 2, 5 * block - 17, 128, block, "bf16", 0.9, wid=410 + block)
    q, k, v = _inputs(w)
    nb = w.num_blocks
    rng = np.random.default_rng(4)
    mask = (rng.random((1, 2, nb, nb)) < 0.6).astype(np.uint8)
    mask[0, 0, 1] = 0
    mask[0, 0, 1, 3] = 1                           # only a future block
    mask[0, 1, 0] = 0
    mask[0, 1, 0, [0, nb - 1]] = 1                 # the diagonal and the ragged tail
    row_cnt = mask.sum(-1).astype(np.int32)
    row_idx = np.zeros((1, 2, nb, nb), dtype=np.int32)
    for h, i in itertools.product(range(2), range(nb)):
        sel = np.nonzero(mask[0, h, i])[0]
        row_idx[0, h, i, :sel.size] = sel
    o, lse = tbs.sparse_fwd(q, k, v, torch.from_numpy(row_cnt).to(DEV), torch.from_numpy(row_idx).to(DEV),
                            block, causal=True)
    torch.cuda.synchronize()
    rows = slice(block, 2 * block)
    assert (o[0, 0, rows] == 0).all() and torch.isneginf(lse[0, 0, rows]).all()
    past = mask * np.tril(np.ones((nb, nb), dtype=np.uint8))
    units = [(0, h, i) for h in range(2) for i in range(nb) if past[0, h, i].any()]
    compare_units(o, lse, q, k, v, block, units, past, q.dtype, causal=True)


def test_causal_full_size_video_sample():
    # The video workload's shape with causal routing: whole mask against the
    # oracle, attention on sampled query blocks (first, last, heaviest, random).
    w = WORKLOADS["video-32k"]
    q, k, v = _inputs(w)
    pr, ws, r, wl, o, lse = _causal_path(w, q, k, v)
    print("  gpu done; oracle routing", flush=True)
    ref = oracle_route_per_head(q, k, w.block, w.top_p, causal=True)
    cmp = compare_route(r, ref)
    rc = r.row_cnt.cpu().numpy()
    nb = pr.num_blocks
    density = rc.sum() / (pr.batch * pr.heads * nb * (nb + 1) / 2)
    print(f"  mask ok (ambiguous mismatches {cmp['ambiguous_mismatches']}), causal density {density:.3f}",
          flush=True)
    rng = np.random.default_rng(6)
    units = []
    for h in range(0, w.heads, 3):
        cand = {0, nb - 1, int(np.argmax(rc[0, h])), int(rng.integers(nb))}
        units += [(0, h, i) for i in sorted(cand)]
    units = routed_units(units, cmp)
    e, le = compare_units(o, lse, q, k, v, w.block, units, cmp["gpu_mask"], q.dtype, causal=True)
    print(f"  {len(units)} sampled blocks: max |O err| {e:.3e}, |LSE err| {le:.3e}", flush=True)


SPLIT = [
    custom_workload(1, 2, 4096, 128, 64, "bf16", 1.0, structured=False, wid=421),   # the dense-4k shape, two heads
    custom_workload(1, 3, 3000, 128, 128, "bf16", 1.0, wid=422),                     # block 128, tail 56
    custom_workload(2, 1, 2500, 64, 64, "bf16", 1.0, wid=423),                       # d = 64, two batches
]


@pytest.mark.parametrize("w", SPLIT, ids=lambda w: w.name)
def test_dense_causal_split_items_match_oracle(w):
    # Few work items: the dense causal kernel runs the longest items as parts
    # of 16 key tiles and merges their partial softmax results.  The route
    # call before it leaves its pooled data in the same workspace region, so
    # the part counters must not rely on the workspace being zero.
    assert dense_causal_splits(w)
    q, k, v = _inputs(w, seed=3)
    pr = tbs.make_problem(q, w.block, causal=True)
    ws = tbs.workspace(pr, DEV)
    tbs.route(q, k, 0.9, w.block, ws=ws, causal=True)
    o, lse = tbs.dense_fwd(q, k, v, w.block, causal=True, ws=ws)
    torch.cuda.synchronize()
    nb = pr.num_blocks
    units = [(b, h, i) for b in range(w.batch) for h in range(w.heads) for i in range(nb)]
    e, le = compare_units(o, lse, q, k, v, w.block, units, None, q.dtype, causal=True)
    print(f"  max |O err| {e:.3e}  max |LSE err| {le:.3e} over {len(units)} blocks", flush=True)
    # the same bits on a second call
    o2, lse2 = tbs.dense_fwd(q, k, v, w.block, causal=True, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)



def test_split_accounting_matches_the_rule():
    # attn_num_workers and attn_workspace_bytes of a split dense causal
    # problem follow the documented rule: parts of at most
    # max(16, ceil(mean tiles per CU / 2)) tiles, equal parts per item, a
    # slot of 256 * d + 1024 floats per queue entry (O of 256 rows, a maximum
    # and a sum per lane of 8 waves) after 256-byte aligned part counters.
    w = SPLIT[0]
    q = torch.empty((w.batch, w.heads, w.seq_len, w.head_dim), dtype=torch.bfloat16, device=DEV)
    pr = tbs.make_problem(q, w.block, causal=True)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    ng = -(-w.seq_len // 256)
    tiles = [-(-min(w.seq_len, 256 * (gi + 1)) // 64) for gi in range(ng)]
    bh = w.batch * w.heads
    part = max(16, (-(-(bh * sum(tiles)) // cus) + 1) // 2)
    entries = bh * sum(-(-t // part) for t in tiles)
    assert tbs.num_workers(pr, tbs.OP_DENSE_FWD) == min(cus, entries)
    counters = -(-(bh * ng * 4) // 256) * 256
    slot = (256 * w.head_dim + 1024) * 4
    assert entries <= bh * ng + 2 * cus
    assert tbs.workspace_bytes(pr, tbs.OP_DENSE_FWD) == 256 + counters + entries * slot
    # non-causal: no split, the control block only
    prn = tbs.make_problem(q, w.block)
    assert tbs.workspace_bytes(prn, tbs.OP_DENSE_FWD) == 256
    assert tbs.num_workers(prn, tbs.OP_DENSE_FWD) == min(cus, bh * ng)
