"""Sparse work items split along their union of key tiles (problems with few
work items): results against the fp64 oracle on every block, against the
unsplit call (ATTN_FLAG_NO_SPLIT) to rounding, and a second call bit for bit;
causal, mixed block sizes, fp8, empty rows; equal items that fill the compute
units are not split.  Every call goes through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from oracle import fp8 as ofp8
import top_block_sparse_pool_amd as tbs
from parity import compare_route, compare_units, oracle_route_per_head, to64
from workloads import custom_workload, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(w, seed=0):
    print(f"[case] {w.describe()} seed={seed}", flush=True)
    return [t.to(DEV) for t in make_inputs(w, seed)]


SPLIT_CASES = [
    (custom_workload(1, 2, 8192, 128, 64, "bf16", 0.9, wid=601), None, False),     # 64 items, 128 key blocks
    (custom_workload(1, 3, 6000, 128, 64, "bf16", 0.95, wid=602), None, True),     # causal, ragged tail
    (custom_workload(1, 2, 7000, 128, 128, "bf16", 0.9, wid=603), 64, False),      # 128-row blocks over 64 keys
    (custom_workload(1, 2, 5000, 64, 64, "bf16", 0.9, wid=604), None, False),      # head_dim 64
]


@pytest.mark.parametrize("w,kb,causal", SPLIT_CASES, ids=lambda x: getattr(x, "name", str(x)))
def test_split_sparse_matches_oracle_and_unsplit(w, kb, causal):
    q, k, v = _inputs(w)
    pr = tbs.make_problem(q, w.block, causal=causal, key_block=kb)
    assert pr.items < 4 * torch.cuda.get_device_properties(0).multi_processor_count
    ws = tbs.workspace(pr, DEV)
    r = tbs.route(q, k, w.top_p, w.block, ws=ws, causal=causal, key_block=kb)
    wl = tbs.schedule(pr, r.row_cnt, ws)
    o, lse = tbs.sparse_fwd(q, k, v, r.row_cnt, r.row_idx, w.block, work_list=wl, ws=ws, causal=causal,
                            key_block=kb)
    o2, lse2 = tbs.sparse_fwd(q, k, v, r.row_cnt, r.row_idx, w.block, work_list=wl, ws=ws, causal=causal,
                              key_block=kb)
    o_ns, lse_ns = tbs.sparse_fwd(q, k, v, r.row_cnt, r.row_idx, w.block, work_list=wl, ws=ws, causal=causal,
                                  key_block=kb, flags=tbs.FLAG_NO_SPLIT)
    o_nat, lse_nat = tbs.sparse_fwd(q, k, v, r.row_cnt, r.row_idx, w.block, ws=ws, causal=causal, key_block=kb)
    torch.cuda.synchronize()
    # deterministic: a second call, and natural item order, give the same bits
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    assert torch.equal(o, o_nat) and torch.equal(lse, lse_nat)
    # the split call merged parts (its rounding differs from the whole items somewhere)
    assert not (torch.equal(o, o_ns) and torch.equal(lse, lse_ns))
    assert (o.float() - o_ns.float()).abs().max().item() <= 2e-2
    fin = torch.isfinite(lse_ns)
    assert torch.equal(fin, torch.isfinite(lse))
    assert (lse[fin] - lse_ns[fin]).abs().max().item() <= 2e-3
    # every block against the oracle, on the GPU's own mask
    ref = oracle_route_per_head(q, k, w.block, w.top_p, causal=causal, key_block=kb)
    cmp = compare_route(r, ref)
    units = [(0, h, i) for h in range(w.heads) for i in range(pr.num_blocks)]
    e, le = compare_units(o, lse, q, k, v, w.block, units, cmp["gpu_mask"], q.dtype, causal=causal, key_block=kb)
    print(f"  {len(units)} blocks: max |O err| {e:.3e}, |LSE err| {le:.3e}", flush=True)


def test_split_fp8_matches_oracle_on_dequantised():
    w = custom_workload(1, 2, 8192, 128, 64, "bf16", 0.9, wid=605)
    q, k, v = _inputs(w)
    pr = tbs.make_problem(q, w.block)
    ws = tbs.workspace(pr, DEV)
    r, qk = tbs.route_fp8(q, k, w.top_p, w.block, ws=ws)
    wl = tbs.schedule(pr, r.row_cnt, ws)
    o, lse = tbs.sparse_fwd_fp8(qk, v, r.row_cnt, r.row_idx, w.block, work_list=wl, ws=ws)
    o2, lse2 = tbs.sparse_fwd_fp8(qk, v, r.row_cnt, r.row_idx, w.block, work_list=wl, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    ref_q = ofp8.quantize_qk(to64(q), to64(k))
    assert np.array_equal(qk.q8.cpu().numpy(), ref_q.q_codes)
    ref = oracle_route_per_head(q, k, w.block, w.top_p)
    cmp = compare_route(r, ref)
    units = [(0, h, i) for h in range(w.heads) for i in range(pr.num_blocks)]
    e, le = compare_units(o, lse, ref_q.q_deq, ref_q.k_deq, v, w.block, units, cmp["gpu_mask"], q.dtype)
    print(f"  fp8 split: max |O err| {e:.3e}, |LSE err| {le:.3e}", flush=True)


def test_split_with_empty_rows_and_hand_made_lists():
    # Rows without blocks (O = 0, LSE = -inf) beside long rows that split.
    w = custom_workload(1, 2, 8192, 128, 64, "bf16", 0.9, wid=606)
    q, k, v = _inputs(w)
    nb = w.num_blocks
    rng = np.random.default_rng(7)
    mask = (rng.random((1, 2, nb, nb)) < 0.6).astype(np.uint8)
    mask[0, 0, :8] = 0                  # two whole work items without keys
    mask[0, 1, 5] = 0
    cnt = torch.tensor(mask.sum(-1), dtype=torch.int32, device=DEV)
    idx = np.zeros((1, 2, nb, nb), dtype=np.int32)
    for h in range(2):
        for i in range(nb):
            sel = np.nonzero(mask[0, h, i])[0]
            idx[0, h, i, : sel.size] = sel
    idx_t = torch.tensor(idx, device=DEV)
    o, lse = tbs.sparse_fwd(q, k, v, cnt, idx_t, w.block)
    torch.cuda.synchronize()
    assert (o[0, 0, : 8 * 64] == 0).all() and torch.isneginf(lse[0, 0, : 8 * 64]).all()
    assert (o[0, 1, 5 * 64: 6 * 64] == 0).all() and torch.isneginf(lse[0, 1, 5 * 64: 6 * 64]).all()
    units = [(0, h, i) for h in range(2) for i in range(0, nb, 3)]
    e, le = compare_units(o, lse, q, k, v, w.block, units, mask, q.dtype)
    print(f"  hand-made lists: max |O err| {e:.3e}", flush=True)


def test_equal_items_filling_the_compute_units_are_not_split():
    # p = 1 and one item of equal length per compute unit or more: no item is
    # longer than the mean work per compute unit, so the call equals the dense
    # call bit for bit without any flag.
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    heads = -(-cus // 16)                       # 16 items of 256 rows per head at N = 4096
    w = custom_workload(1, heads, 4096, 128, 64, "bf16", 1.0, structured=False, wid=607)
    q, k, v = _inputs(w)
    pr = tbs.make_problem(q, w.block)
    ws = tbs.workspace(pr, DEV)
    r = tbs.route(q, k, 1.0, w.block, ws=ws)
    o, lse = tbs.sparse_fwd(q, k, v, r.row_cnt, r.row_idx, w.block, ws=ws)
    od, lsed = tbs.dense_fwd(q, k, v, w.block, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(o, od) and torch.equal(lse, lsed)
