"""attn_sparse_fwd_noalloc (no workspace; the queue counters live in the
library's static per-GPU scratch) against attn_sparse_fwd through the C ABI:
two calls in a row, the second on a smaller input, and a causal call after
them.  The allocation-free call never splits a work item along its keys, so
it is compared with attn_sparse_fwd given ATTN_FLAG_NO_SPLIT: outputs must be
equal bit for bit (same kernel, same work list); against the default call,
which may split few-item problems, they agree to rounding."""
import pytest
import torch

import top_block_sparse_pool_amd as tbs
from workloads import custom_workload, make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _case(w, causal=False):
    print(f"[case] noalloc {w.describe()} causal={causal}", flush=True)
    q, k, v = [t.to(DEV) for t in make_inputs(w, 0)]
    pr = tbs.make_problem(q, w.block, causal=causal)
    ws = tbs.workspace(pr, DEV)
    r = tbs.route(q, k, w.top_p, w.block, ws=ws, causal=causal)
    wl = tbs.schedule(pr, r.row_cnt, ws)
    o_ref, lse_ref = tbs.sparse_fwd(q, k, v, r.row_cnt, r.row_idx, w.block, work_list=wl, ws=ws, causal=causal,
                                    flags=tbs.FLAG_NO_SPLIT)
    o_def, lse_def = tbs.sparse_fwd(q, k, v, r.row_cnt, r.row_idx, w.block, work_list=wl, ws=ws, causal=causal)
    o = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), device=DEV)
    tbs.sparse_fwd_noalloc(q, k, v, r.row_cnt, r.row_idx, w.block, work_list=wl, o=o, lse=lse, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref), f"O differs: max {(o.float() - o_ref.float()).abs().max().item()}"
    assert torch.equal(lse, lse_ref)
    assert (o.float() - o_def.float()).abs().max().item() <= 2e-2
    fin = torch.isfinite(lse_ref)
    assert torch.equal(fin, torch.isfinite(lse_def))
    assert (lse[fin] - lse_def[fin]).abs().max().item() <= 2e-3
    # natural order (no work list) gives the same bits as well
    o2 = torch.full_like(q, float("nan"))
    tbs.sparse_fwd_noalloc(q, k, v, r.row_cnt, r.row_idx, w.block, o=o2, want_lse=False, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o2, o_ref)


def test_noalloc_equals_workspace_call_twice_then_smaller():
    _case(custom_workload(1, 8, 4000, 128, 64, "bf16", 0.9, wid=801))      # 63 blocks, ragged tail
    _case(custom_workload(1, 2, 1000, 64, 64, "bf16", 0.8, wid=802))       # smaller, d = 64
    _case(custom_workload(1, 3, 1500, 128, 128, "bf16", 0.9, wid=803), causal=True)
