"""GPU edge cases against the fp64 oracle: exact ties and near ties (equal
to 2^-24 relative) in the block probabilities,
the largest sizes the C ABI accepts (1024 key blocks for routing, 2048 for
the sparse forward), and p so small that every row keeps one block.  Every
call goes through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import top_block_sparse_pool_amd as tbs
from parity import compare_route, compare_units, oracle_route_per_head, routed_units, to64
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


def _ranked_correctly(r, nv_of=None):
    """Every row's selection ascending, then its ranked tail by (P desc, index asc)
    on the GPU's own probabilities; the selection is a prefix of that order."""
    prob = r.block_prob.cpu().numpy()
    rc, ri = r.row_cnt.cpu().numpy(), r.row_idx.cpu().numpy()
    B, H, nb, nbk = prob.shape
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                nv = nbk if nv_of is None else nv_of(i)
                kk = int(rc[b, h, i])
                sel, tail = ri[b, h, i, :kk], ri[b, h, i, kk:nv]
                assert (np.diff(sel) > 0).all()
                order = sorted(range(nv), key=lambda j: (-prob[b, h, i, j], j))
                assert sorted(sel.tolist()) == sorted(order[:kk])
                assert tail.tolist() == order[kk:]


@pytest.mark.parametrize("nb", [64, 512, 1000])   # 1000: rows of more than 512 blocks (rolled sort stages)
def test_near_ties_ranked_exactly(nb):
    # Every query token is the same vector a, and key block 2t+1 is block 2t
    # with one element one fp32 ulp larger where a is positive: the pair's
    # probabilities differ by about 1e-10 relative (the same high bits of
    # the double), the larger index larger, so the ranking must put the odd
    # block first.  fp32 inputs, so the ulp survives.
    d, block = 64, 64
    N = nb * block
    g = torch.Generator().manual_seed(5)
    a = torch.rand(d, generator=g) + 0.5
    q = a.expand(1, 1, N, d).contiguous()
    kb = torch.randn(1, 1, nb // 2, block, d, generator=g) * 2
    k = torch.empty(1, 1, nb, block, d)
    k[:, :, 0::2] = kb
    k[:, :, 1::2] = kb
    k[:, :, 1::2, 0, 0] = torch.nextafter(kb[:, :, :, 0, 0], torch.tensor(float("inf")))
    k = k.reshape(1, 1, N, d)
    q, k = q.to(DEV), k.to(DEV)
    r = tbs.route(q, k, 0.5, block, return_prob=True)
    torch.cuda.synchronize()
    prob = r.block_prob.cpu().numpy()[0, 0, 0]
    assert (prob[1::2] > prob[0::2]).all()
    rel = (prob[1::2] - prob[0::2]) / prob[0::2]
    print(f"  relative gap of the planted pairs: {rel.min():.2e} .. {rel.max():.2e}", flush=True)
    assert rel.max() < 2.0 ** -24
    _ranked_correctly(r)
    ref = oracle_route_per_head(q, k, block, 0.5)
    compare_route(r, ref)


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
    units = routed_units([(0, h, i) for h in range(2) for i in (0, 511, 1023)], cmp)
    e, le = compare_units(o, lse, q, k, v, w.block, units, cmp["gpu_mask"], q.dtype)
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


@pytest.mark.parametrize("block,kb,causal", [(64, 64, True), (128, 64, False), (128, 64, True)],
                         ids=["64-64-causal", "128-64", "128-64-causal"])
def test_long_rows_route_and_sampled_attention(block, kb, causal):
    # 700 key blocks (more than 512: the selection runs its rolled sort
    # stages), with causal eligibility (row i ranks only its eligible
    # blocks) and with 128-row query blocks over 64-key blocks; ragged tail.
    N = 700 * 64 - 30
    w = custom_workload(1, 2, N, 128, block, "bf16", 0.9, wid=720 + block + (1 if causal else 0))
    q, k, v = _inputs(w)
    pr = tbs.make_problem(q, block, causal=causal, key_block=kb)
    assert pr.num_key_blocks == 700
    ws = tbs.workspace(pr, DEV)
    r = tbs.route(q, k, w.top_p, block, ws=ws, causal=causal, key_block=kb, return_prob=True)
    wl = tbs.schedule(pr, r.row_cnt, ws)
    o, lse = tbs.sparse_fwd(q, k, v, r.row_cnt, r.row_idx, block, work_list=wl, ws=ws, causal=causal,
                            key_block=kb)
    torch.cuda.synchronize()
    nb, nbk = pr.num_blocks, pr.num_key_blocks
    ref = oracle_route_per_head(q, k, block, w.top_p, causal=causal, key_block=kb)
    cmp = compare_route(r, ref)
    print(f"  ambiguous mismatches {cmp['ambiguous_mismatches']}", flush=True)
    elig = oracle.causal_eligible(nb, nbk, block, kb) if causal else None
    _ranked_correctly(r, None if elig is None else (lambda i: int(elig[i])))
    rc = r.row_cnt.cpu().numpy()
    rng = np.random.default_rng(11)
    units = []
    for h in range(pr.heads):
        cand = {0, nb - 1, int(np.argmax(rc[0, h])), int(rng.integers(nb)), int(rng.integers(nb))}
        units += [(0, h, i) for i in sorted(cand)]
    units = routed_units(units, cmp)
    e, le = compare_units(o, lse, q, k, v, block, units, cmp["gpu_mask"], q.dtype, causal=causal, key_block=kb)
    print(f"  {len(units)} sampled blocks: max |O err| {e:.3e}, |LSE err| {le:.3e}", flush=True)
