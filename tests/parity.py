"""Comparison helpers for the GPU parity tests (test infrastructure).

Routing: the GPU mask must equal the oracle mask everywhere except on blocks
the oracle marks ambiguous (within 1e-5 of the top-p cut); such mismatches are
counted and returned.  Rows whose masks agree must also agree exactly on the
row count and the ascending index list.

Attention: GPU outputs (bf16 or fp32, upcast exactly) are compared element by
element with the fp64 oracle evaluated on the GPU's own mask (which equals the
oracle's mask except inside the window, so a row whose selection differs by an
ambiguous block is still checked, against the attention its selection defines):
max abs error <= 2e-2 for bf16 inputs and <= 1e-4 for fp32 inputs.  LSE uses
2e-3 / 1e-4; a query without allowed keys must be -inf on both sides (and O = 0).
Sampled units are extended by every query block whose mask row differs from the
oracle's (routed_units).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

WINDOW = 1e-5
O_TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-4}
LSE_TOL = {torch.bfloat16: 2e-3, torch.float32: 1e-4}


def to64(t) -> np.ndarray:
    if isinstance(t, np.ndarray):
        return t.astype(np.float64, copy=False)
    return t.detach().to("cpu").to(torch.float64).numpy()


def oracle_route_per_head(q: torch.Tensor, k: torch.Tensor, block: int, top_p: float, scale=None, causal=False,
                          key_block=None):
    """Oracle routing head by head (bounded host memory at full sizes).

    Returns mask, row_cnt, row_idx, head_cnt and the ambiguity map, [B,H,...].
    """
    B, H, N, d = q.shape
    nb = -(-N // block)
    nbk = -(-N // (key_block or block))
    mask = np.zeros((B, H, nb, nbk), dtype=np.uint8)
    amb = np.zeros((B, H, nb, nbk), dtype=bool)
    row_cnt = np.zeros((B, H, nb), dtype=np.int64)
    row_idx = np.full((B, H, nb, nbk), -1, dtype=np.int32)
    for b in range(B):
        for h in range(H):
            r = oracle.route(to64(q[b:b + 1, h:h + 1]), to64(k[b:b + 1, h:h + 1]), block, top_p, scale,
                             causal=causal, key_block=key_block)
            mask[b, h] = r.mask[0, 0]
            row_cnt[b, h] = r.row_cnt[0, 0]
            row_idx[b, h] = r.row_idx[0, 0]
            amb[b, h] = oracle.ambiguous_blocks(r, WINDOW)[0, 0]
    return dict(mask=mask, row_cnt=row_cnt, row_idx=row_idx, head_cnt=row_cnt.sum(-1), amb=amb)


def compare_route(gpu_route, ref) -> dict:
    """Assert routing parity; return {'rows_agree': bool[B,H,nb], 'ambiguous_mismatches': int}."""
    mask = gpu_route.mask.cpu().numpy()
    diff = mask != ref["mask"]
    bad = diff & ~ref["amb"]
    assert not bad.any(), f"{int(bad.sum())} mask mismatches outside the 1e-5 window, first at {np.argwhere(bad)[:5]}"
    rows_agree = ~diff.any(-1)
    rc = gpu_route.row_cnt.cpu().numpy().astype(np.int64)
    assert (rc[rows_agree] == ref["row_cnt"][rows_agree]).all(), "row counts differ on agreeing rows"
    assert (rc == mask.astype(np.int64).sum(-1)).all(), "row counts disagree with the GPU mask"
    ri = gpu_route.row_idx.cpu().numpy()
    nb = mask.shape[-1]
    valid = np.arange(nb)[None, None, None, :] < rc[..., None]
    want = np.where(valid, ref["row_idx"], -1)
    got = np.where(valid, ri, -1)
    assert (got[rows_agree] == want[rows_agree]).all(), "index lists differ on agreeing rows"
    hc = gpu_route.head_cnt.cpu().numpy().astype(np.int64)
    assert (hc == rc.sum(-1)).all(), "head counts are not the sum of row counts"
    return dict(rows_agree=rows_agree, ambiguous_mismatches=int(diff.sum()), gpu_mask=mask)


def routed_units(units, cmp) -> list:
    """`units` plus every query block whose GPU mask row differs from the oracle's."""
    extra = {tuple(int(x) for x in u) for u in np.argwhere(~cmp["rows_agree"])}
    return sorted({tuple(int(x) for x in u) for u in units} | extra)


def compare_units(o_gpu, lse_gpu, q, k, v, block, units, mask, dtype, scale=None, causal=False, key_block=None):
    """Compare GPU output rows of `units` with the oracle, head by head.

    Returns (max_o_err, max_lse_err)."""
    N = q.shape[2]
    by_head = {}
    for (b, h, i) in units:
        by_head.setdefault((b, h), []).append(i)
    emax = lmax = 0.0
    for (b, h), blocks in sorted(by_head.items()):
        sl = (slice(b, b + 1), slice(h, h + 1))
        m = None if mask is None else mask[b:b + 1, h:h + 1]
        ref = oracle.attend_units(to64(q[sl]), to64(k[sl]), to64(v[sl]), block, [(0, 0, i) for i in blocks],
                                  mask=m, scale=scale, causal=causal, key_block=key_block)
        o64 = to64(o_gpu[sl])[0, 0]
        l64 = to64(lse_gpu[sl])[0, 0] if lse_gpu is not None else None
        for (_, _, i), (ro, rl) in ref.items():
            lo, hi = i * block, min(N, (i + 1) * block)
            emax = max(emax, float(np.max(np.abs(o64[lo:hi] - ro))))
            if l64 is not None:
                gl, ol = l64[lo:hi], rl
                both_empty = np.isneginf(gl) & np.isneginf(ol)          # queries without keys: -inf on both sides
                d = np.where(both_empty, 0.0, np.abs(np.where(both_empty, 0.0, gl) - np.where(both_empty, 0.0, ol)))
                lmax = max(lmax, float(np.max(d)))
    assert emax <= O_TOL[dtype], f"max |O - O_ref| = {emax:.3e} > {O_TOL[dtype]}"
    if lse_gpu is not None:
        assert lmax <= LSE_TOL[dtype], f"max |LSE - LSE_ref| = {lmax:.3e} > {LSE_TOL[dtype]}"
    return emax, lmax


def dense_causal_splits(w) -> bool:
    """Whether attn_dense_fwd(causal) splits this bf16 workload's work items
    along the keys: fewer than four items of 256 query rows per compute unit,
    and a last item longer than half the mean work per compute unit (at
    least 16 key tiles of 64 keys)."""
    if w.dtype != "bf16":
        return False
    ng = -(-w.seq_len // 256)
    items = w.batch * w.heads * ng
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tiles = [-(-min(w.seq_len, 256 * (gi + 1)) // 64) for gi in range(ng)]
    mean = -(-(w.batch * w.heads * sum(tiles)) // cus)
    part = max(16, (mean + 1) // 2)
    return items < 4 * cus and tiles[-1] > part
