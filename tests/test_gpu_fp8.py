"""GPU parity of the FP8 (E4M3) path: the quantiser against the oracle's
quantiser bit for bit (codes, signs of zero and fp32 scales), and the fp8
attention kernels against the fp64 oracle attention on the dequantised Q and K
(the bf16 tolerance: the products of codes are exact and V, P and O are as in
the bf16 path).  Also: p = 1 sparse equals dense bit for bit, causal and mixed
block sizes, and a bound on the effect of quantisation itself.  Every call
goes through the C ABI."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8 as ofp8
import top_block_sparse_pool_amd as tbs
from parity import compare_route, compare_units, oracle_route_per_head, to64, dense_causal_splits
from workloads import WORKLOADS, custom_workload, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = [
    custom_workload(1, 3, 1000, 128, 64, "bf16", 0.9, wid=501),     # nb 16, tail 40
    custom_workload(2, 2, 1500, 128, 128, "bf16", 0.8, wid=502),    # two key tiles per block, tail 92
    custom_workload(1, 2, 1300, 128, 128, "bf16", 0.95, wid=503),   # tail 20
    custom_workload(1, 2, 64, 128, 64, "bf16", 0.5, wid=504),       # a single block
    custom_workload(1, 1, 5, 128, 64, "bf16", 0.9, wid=505),        # N < block
]


def _inputs(w, seed=0):
    print(f"[case] fp8 {w.describe()} seed={seed}", flush=True)
    return [t.to(DEV) for t in make_inputs(w, seed)]


def _check_quantised(qk, q, k):
    ref = ofp8.quantize_qk(to64(q), to64(k))
    q8, k8 = qk.q8.cpu().numpy(), qk.k8.cpu().numpy()
    bad_q = np.argwhere(q8 != ref.q_codes)
    bad_k = np.argwhere(k8 != ref.k_codes)
    assert bad_q.size == 0, f"{len(bad_q)} Q codes differ, first {bad_q[:3]}: gpu {q8[tuple(bad_q[0])]:#x} " \
                            f"oracle {ref.q_codes[tuple(bad_q[0])]:#x}"
    assert bad_k.size == 0, f"{len(bad_k)} K codes differ, first {bad_k[:3]}"
    np.testing.assert_array_equal(qk.q_scale.cpu().numpy().view(np.uint32), ref.q_scale.view(np.uint32))
    np.testing.assert_array_equal(qk.k_scale.cpu().numpy().view(np.uint32), ref.k_scale.view(np.uint32))
    return ref


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_quantize_matches_oracle_bitwise(w):
    q, k, _ = _inputs(w)
    qk = tbs.quantize_qk_fp8(q, k, w.block)
    torch.cuda.synchronize()
    _check_quantised(qk, q, k)


def test_quantize_special_values(golden_dir):
    # The hand-worked rows (fp32 and E4M3 ties, negative zero), zero tokens, a
    # zero key tile, and values far below their group maximum (subnormal codes).
    with open(os.path.join(golden_dir, "e4m3_quant_example.json")) as f:
        g = json.load(f)
    print("[case] fp8 quantiser special values", flush=True)
    B, H, N, d = 1, 2, 200, 128
    rng = np.random.default_rng(7)
    q = torch.from_numpy(rng.standard_normal((B, H, N, d))).to(torch.bfloat16)
    k = torch.from_numpy(rng.standard_normal((B, H, N, d))).to(torch.bfloat16)
    for t, r in enumerate(g["rows"]):
        q[0, 0, t] = 0
        q[0, 0, t, :len(r["x"])] = torch.tensor(r["x"], dtype=torch.float64).to(torch.bfloat16)
    q[0, 1, 3] = 0                                   # a zero token
    k[0, 1, 64:128] = 0                              # a zero key tile
    q[0, 1, 4, 1:] *= 2.0 ** -12                     # one large value, the rest near or below 2^-6 * scale
    q[0, 1, 4, 0] = 4.0
    k[0, 0, 130, :] *= 2.0 ** -12                    # a tiny row inside a normal tile
    k[0, 0, 131, 5] = 60.0
    q, k = q.to(DEV), k.to(DEV)
    qk = tbs.quantize_qk_fp8(q, k, 64)
    torch.cuda.synchronize()
    ref = _check_quantised(qk, q, k)
    for t, r in enumerate(g["rows"]):
        assert qk.q8[0, 0, t, :len(r["codes"])].cpu().tolist() == r["codes"], r["name"]
    assert (qk.k8[0, 1, 64:128] == 0).all() and qk.k_scale[0, 1, 1].item() == 0.0
    sub = ref.q_codes[0, 1, 4, 1:]
    assert (((sub & 0x78) == 0) & ((sub & 0x07) != 0)).any(), "expected subnormal codes in the test input"


def _fp8_path(w, q, k, v, top_p=None, causal=False, key_block=None, ws=None, flags=0):
    p = w.top_p if top_p is None else top_p
    pr = tbs.make_problem(q, w.block, causal=causal, key_block=key_block)
    ws = tbs.workspace(pr, DEV) if ws is None else ws
    r = tbs.route(q, k, p, w.block, ws=ws, causal=causal, key_block=key_block)
    wl = tbs.schedule(pr, r.row_cnt, ws)
    qk = tbs.quantize_qk_fp8(q, k, w.block, key_block=key_block)
    o, lse = tbs.sparse_fwd_fp8(qk, v, r.row_cnt, r.row_idx, w.block, work_list=wl, ws=ws, causal=causal,
                                key_block=key_block, flags=flags)
    torch.cuda.synchronize()
    return pr, ws, r, qk, o, lse


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_sparse_fp8_matches_oracle_on_dequantised(w, causal):
    q, k, v = _inputs(w)
    pr, ws, r, qk, o, lse = _fp8_path(w, q, k, v, causal=causal)
    ref_q = _check_quantised(qk, q, k)
    ref = oracle_route_per_head(q, k, w.block, w.top_p, causal=causal)
    cmp = compare_route(r, ref)
    units = [(b, h, i) for b in range(w.batch) for h in range(w.heads) for i in range(pr.num_blocks)]
    e, le = compare_units(o, lse, ref_q.q_deq, ref_q.k_deq, v, w.block, units, cmp["gpu_mask"], q.dtype,
                          causal=causal)
    print(f"  {len(units)} blocks: max |O err| {e:.3e}, |LSE err| {le:.3e}", flush=True)


@pytest.mark.parametrize("kb", [(128, 64), (64, 128)], ids=["q128k64", "q64k128"])
def test_sparse_fp8_mixed_blocks(kb):
    block, key_block = kb
    w = custom_workload(1, 2, 1100, 128, block, "bf16", 0.85, wid=510 + block // 64)
    q, k, v = _inputs(w)
    for causal in (False, True):
        pr, ws, r, qk, o, lse = _fp8_path(w, q, k, v, causal=causal, key_block=key_block)
        ref_q = _check_quantised(qk, q, k)
        ref = oracle_route_per_head(q, k, block, w.top_p, causal=causal, key_block=key_block)
        cmp = compare_route(r, ref)
        units = [(0, h, i) for h in range(w.heads) for i in range(pr.num_blocks)]
        e, le = compare_units(o, lse, ref_q.q_deq, ref_q.k_deq, v, block, units, cmp["gpu_mask"], q.dtype,
                              causal=causal, key_block=key_block)
        print(f"  causal={causal}: {len(units)} blocks, max |O err| {e:.3e}, |LSE err| {le:.3e}", flush=True)


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("w", CASES[:3], ids=lambda w: w.name)
def test_dense_fp8_equals_sparse_at_p1(w, causal):
    q, k, v = _inputs(w, seed=1)
    ns = tbs.FLAG_NO_SPLIT   # both calls run every work item whole
    pr, ws, r, qk, o_s, l_s = _fp8_path(w, q, k, v, top_p=1.0, causal=causal, flags=ns)
    o_d, l_d = tbs.dense_fwd_fp8(qk, v, w.block, causal=causal, ws=ws, flags=ns)
    torch.cuda.synchronize()
    assert torch.equal(o_s, o_d) and torch.equal(l_s, l_d)
    o_d, l_d = tbs.dense_fwd_fp8(qk, v, w.block, causal=causal, ws=ws)
    torch.cuda.synchronize()
    if not (causal and dense_causal_splits(w)):
        assert torch.equal(o_s, o_d) and torch.equal(l_s, l_d)
    else:
        # split items along the keys: equal to rounding (both checked against the oracle below)
        assert (o_d.float() - o_s.float()).abs().max().item() <= 2e-2
        assert (l_d - l_s).abs().max().item() <= 2e-3
    ref_q = ofp8.quantize_qk(to64(q), to64(k))
    units = [(b, h, i) for b in range(w.batch) for h in range(w.heads) for i in range(pr.num_blocks)]
    compare_units(o_d, l_d, ref_q.q_deq, ref_q.k_deq, v, w.block, units, None, q.dtype, causal=causal)


def test_quantisation_effect_is_bounded():
    # Against exact attention on the unquantised inputs the fp8 output differs
    # by the softmax's response to the logit errors: with delta_t the largest
    # |logit error| of query t (computed in fp64 from the oracle's dequantised
    # operands), the weights move by at most e^(2 delta_t) - 1 in l1 norm, so
    # |O_fp8 - O| <= (e^(2 delta_t) - 1) * max |V| + the bf16 tolerance.
    w = CASES[0]
    q, k, v = _inputs(w, seed=2)
    pr, ws, r, qk, o, lse = _fp8_path(w, q, k, v, top_p=1.0)
    ref_q = ofp8.quantize_qk(to64(q), to64(k))
    q64, k64, v64 = to64(q), to64(k), to64(v)
    s = 1.0 / np.sqrt(w.head_dim)
    worst = 0.0
    for h in range(w.heads):
        dl = s * np.abs(ref_q.q_deq[0, h] @ ref_q.k_deq[0, h].T - q64[0, h] @ k64[0, h].T)
        delta = dl.max(axis=1)
        o_ref, _ = oracle.attend(q64[:, h:h + 1], k64[:, h:h + 1], v64[:, h:h + 1], w.block)
        err = np.abs(to64(o)[0, h] - o_ref[0, 0]).max(axis=1)
        bound = np.expm1(2 * delta) * np.abs(v64[0, h]).max() + 2e-2
        assert np.all(err <= bound), f"head {h}: error {err.max():.3e} above its bound"
        worst = max(worst, float(err.max()))
    print(f"  max |O_fp8 - O_exact| = {worst:.3e}", flush=True)


def test_full_size_video_fp8_sampled():
    w = WORKLOADS["video-32k"]
    print(f"[case] fp8 {w.describe()}", flush=True)
    q, k, v = [t.to(DEV) for t in make_inputs(w, 0)]
    pr, ws, r, qk, o, lse = _fp8_path(w, q, k, v)
    print("  gpu done; oracle quantiser and routing", flush=True)
    # Quantiser on two heads, bit for bit.
    for h in (0, w.heads - 1):
        ref = ofp8.quantize_qk(to64(q[:, h:h + 1]), to64(k[:, h:h + 1]))
        assert np.array_equal(qk.q8[:, h:h + 1].cpu().numpy(), ref.q_codes)
        assert np.array_equal(qk.k8[:, h:h + 1].cpu().numpy(), ref.k_codes)
        assert np.array_equal(qk.k_scale[:, h:h + 1].cpu().numpy(), ref.k_scale)
    heads = [0, 13, w.heads - 1]
    rng = np.random.default_rng(11)
    for h in heads:
        sl = slice(h, h + 1)
        ref_q = ofp8.quantize_qk(to64(q[:, sl]), to64(k[:, sl]))
        ref = oracle_route_per_head(q[:, sl], k[:, sl], w.block, w.top_p)
        rc = r.row_cnt[:, sl].cpu().numpy()
        gmask = r.mask[:, sl].cpu().numpy()
        differ = (gmask != ref["mask"]).any(-1)
        assert not ((gmask != ref["mask"]) & ~ref["amb"]).any()
        cand = {int(np.argmax(rc[0, 0])), int(np.argmin(rc[0, 0])), pr.num_blocks - 1}
        cand |= {int(x) for x in rng.integers(0, pr.num_blocks, size=2)}
        cand |= {int(i) for i in np.nonzero(differ[0, 0])[0]}
        units = [(0, 0, i) for i in sorted(cand)]
        e, le = compare_units(o[:, sl], lse[:, sl], ref_q.q_deq, ref_q.k_deq, v[:, sl], w.block, units, gmask,
                              q.dtype)
        print(f"  head {h}: {len(units)} sampled blocks, max |O err| {e:.3e}, |LSE err| {le:.3e}", flush=True)


def test_fp8_processing_order_is_bitwise_invariant():
    # Each work item is computed by one workgroup in a fixed key order, so the
    # natural order, the longest-first list and other head windows give the
    # same bits.
    w = CASES[1]
    q, k, v = _inputs(w, seed=3)
    pr, ws, r, qk, o, lse = _fp8_path(w, q, k, v)
    outs = []
    for hw in (None, 0, 1):
        wl = None if hw is None else tbs.schedule(pr, r.row_cnt, ws, head_window=hw)
        o2, l2 = tbs.sparse_fwd_fp8(qk, v, r.row_cnt, r.row_idx, w.block, work_list=wl, ws=ws)
        outs.append((o2, l2))
    torch.cuda.synchronize()
    for o2, l2 in outs:
        assert torch.equal(o2, o) and torch.equal(l2, lse)


def test_sparse_attention_fp8_wrapper_matches_the_calls():
    w = CASES[0]
    q, k, v = _inputs(w, seed=4)
    o, lse, r, wl = tbs.sparse_attention(q, k, v, w.top_p, w.block, fp8=True)
    pr, ws, r2, qk, o2, l2 = _fp8_path(w, q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(r.mask, r2.mask) and torch.equal(o, o2) and torch.equal(lse, l2)


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_dense_fp8_on_the_dense_workload(causal):
    # dense-4k: iid N(0,1) inputs, H = 16, N = 4096; sampled query blocks of
    # every head against the oracle on the dequantised operands.
    w = WORKLOADS["dense-4k"]
    print(f"[case] fp8 dense {w.describe()} causal={causal}", flush=True)
    q, k, v = [t.to(DEV) for t in make_inputs(w, 0)]
    qk = tbs.quantize_qk_fp8(q, k, w.block)
    o, lse = tbs.dense_fwd_fp8(qk, v, w.block, causal=causal)
    torch.cuda.synchronize()
    ref_q = ofp8.quantize_qk(to64(q), to64(k))
    rng = np.random.default_rng(9)
    units = [(0, h, int(i)) for h in range(w.heads) for i in rng.integers(0, w.num_blocks, size=2)]
    units.append((0, w.heads - 1, w.num_blocks - 1))
    e, le = compare_units(o, lse, ref_q.q_deq, ref_q.k_deq, v, w.block, units, None, q.dtype, causal=causal)
    print(f"  {len(units)} blocks: max |O err| {e:.3e}, |LSE err| {le:.3e}", flush=True)


def test_fp8_after_union_fill():
    # attn_augment_union changes only the lists; the fp8 kernel then runs over
    # the filled lists (every row of an item takes the item's union).
    w = CASES[0]
    q, k, v = _inputs(w, seed=5)
    pr = tbs.make_problem(q, w.block)
    ws = tbs.workspace(pr, DEV)
    r = tbs.route(q, k, w.top_p, w.block, ws=ws)
    tbs.augment_union(pr, r)
    wl = tbs.schedule(pr, r.row_cnt, ws)
    qk = tbs.quantize_qk_fp8(q, k, w.block)
    o, lse = tbs.sparse_fwd_fp8(qk, v, r.row_cnt, r.row_idx, w.block, work_list=wl, ws=ws)
    torch.cuda.synchronize()
    mask = r.mask.cpu().numpy()
    ref_q = ofp8.quantize_qk(to64(q), to64(k))
    units = [(b, h, i) for b in range(w.batch) for h in range(w.heads) for i in range(pr.num_blocks)]
    e, le = compare_units(o, lse, ref_q.q_deq, ref_q.k_deq, v, w.block, units, mask, q.dtype)
    print(f"  {len(units)} blocks over filled lists: max |O err| {e:.3e}", flush=True)


def test_full_size_long_video_fp8_sampled():
    w = WORKLOADS["video-119k"]
    print(f"[case] fp8 {w.describe()}", flush=True)
    q, k, v = [t.to(DEV) for t in make_inputs(w, 0)]
    pr, ws, r, qk, o, lse = _fp8_path(w, q, k, v)
    print("  gpu done; oracle per sampled head", flush=True)
    rng = np.random.default_rng(13)
    for h in (0, w.heads - 1):
        sl = slice(h, h + 1)
        ref = ofp8.quantize_qk(to64(q[:, sl]), to64(k[:, sl]))
        assert np.array_equal(qk.q8[:, sl].cpu().numpy(), ref.q_codes)
        assert np.array_equal(qk.k8[:, sl].cpu().numpy(), ref.k_codes)
        route_ref = oracle_route_per_head(q[:, sl], k[:, sl], w.block, w.top_p)
        gmask = r.mask[:, sl].cpu().numpy()
        differ = (gmask != route_ref["mask"]).any(-1)
        assert not ((gmask != route_ref["mask"]) & ~route_ref["amb"]).any()
        cand = {int(x) for x in rng.integers(0, pr.num_blocks, size=3)} | {pr.num_blocks - 1}
        cand |= {int(i) for i in np.nonzero(differ[0, 0])[0]}
        units = [(0, 0, i) for i in sorted(cand)]
        e, le = compare_units(o[:, sl], lse[:, sl], ref.q_deq, ref.k_deq, v[:, sl], w.block, units, gmask, q.dtype)
        print(f"  head {h}: {len(units)} sampled blocks, max |O err| {e:.3e}, |LSE err| {le:.3e}", flush=True)


ROUTE_FP8_CASES = [
    (custom_workload(1, 3, 1000, 128, 64, "bf16", 0.9, wid=540), None, False),     # ragged tail of 40
    (custom_workload(2, 2, 1300, 128, 128, "bf16", 0.9, wid=541), None, False),    # block 128, tail 20
    (custom_workload(1, 2, 1100, 128, 128, "bf16", 0.85, wid=542), 64, False),     # 128-row blocks over 64 keys
    (custom_workload(1, 2, 1100, 128, 64, "bf16", 0.85, wid=543), 128, True),      # 64 over 128, causal
    (custom_workload(1, 2, 64, 128, 64, "bf16", 0.5, wid=544), None, False),       # one block
    (custom_workload(1, 1, 5, 128, 64, "bf16", 0.9, wid=545), None, True),         # N < block
]


@pytest.mark.parametrize("w,kb,causal", ROUTE_FP8_CASES, ids=lambda x: getattr(x, "name", str(x)))
def test_route_fp8_equals_route_then_quantize(w, kb, causal):
    # One read of Q and K gives the routing of attn_route and the codes of
    # attn_quantize_qk_fp8, bit for bit.
    q, k, v = _inputs(w)
    pr = tbs.make_problem(q, w.block, causal=causal, key_block=kb)
    ws = tbs.workspace(pr, DEV)
    r0 = tbs.route(q, k, w.top_p, w.block, ws=ws, return_prob=True, causal=causal, key_block=kb)
    qk0 = tbs.quantize_qk_fp8(q, k, w.block, key_block=kb)
    torch.cuda.synchronize()
    r1, qk1 = tbs.route_fp8(q, k, w.top_p, w.block, ws=ws, return_prob=True, causal=causal, key_block=kb)
    torch.cuda.synchronize()
    for a, b in [(r0.mask, r1.mask), (r0.row_cnt, r1.row_cnt), (r0.head_cnt, r1.head_cnt),
                 (r0.block_prob, r1.block_prob), (qk0.q8, qk1.q8), (qk0.k8, qk1.k8),
                 (qk0.q_scale, qk1.q_scale), (qk0.k_scale, qk1.k_scale)]:
        assert torch.equal(a, b)
    rc = r0.row_cnt.cpu().numpy()
    valid = np.arange(pr.num_key_blocks)[None, None, None, :] < rc[..., None]
    if not causal:
        assert torch.equal(r0.row_idx, r1.row_idx)
    else:
        assert (np.where(valid, r0.row_idx.cpu().numpy(), -1) == np.where(valid, r1.row_idx.cpu().numpy(), -1)).all()
    # and the routing itself against the oracle
    compare_route(r1, oracle_route_per_head(q, k, w.block, w.top_p, causal=causal, key_block=kb))


def test_route_fp8_full_size_video():
    w = WORKLOADS["video-32k"]
    print(f"[case] route_fp8 {w.describe()}", flush=True)
    q, k, v = [t.to(DEV) for t in make_inputs(w, 0)]
    pr = tbs.make_problem(q, w.block)
    ws = tbs.workspace(pr, DEV)
    r0 = tbs.route(q, k, w.top_p, w.block, ws=ws, return_prob=True)
    qk0 = tbs.quantize_qk_fp8(q, k, w.block)
    torch.cuda.synchronize()
    r1, qk1 = tbs.route_fp8(q, k, w.top_p, w.block, ws=ws, return_prob=True)
    torch.cuda.synchronize()
    for a, b in [(r0.mask, r1.mask), (r0.row_cnt, r1.row_cnt), (r0.row_idx, r1.row_idx), (r0.head_cnt, r1.head_cnt),
                 (r0.block_prob, r1.block_prob), (qk0.q8, qk1.q8), (qk0.k8, qk1.k8), (qk0.q_scale, qk1.q_scale),
                 (qk0.k_scale, qk1.k_scale)]:
        assert torch.equal(a, b)
