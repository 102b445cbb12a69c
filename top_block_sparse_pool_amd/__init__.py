"""Top-p block-sparse attention forward for AMD MI355X (gfx950).

Python binding over the C ABI of ``libattn_tbs.so`` (declared in
``include/attn_tbs.h``).  This layer only marshals arguments: it takes torch
tensors as device memory, passes their pointers and sizes together with the
current HIP stream, and raises on a non-zero status.  Every step of the path
-- pooling, scores, softmax, top-p cut, scheduling and attention -- runs in
the library's HIP kernels; there is no CPU fallback, and calls fail loudly if
the library has not been built.

The four calls of the path (same names as the C ABI):
    route(q, k, top_p, block, causal)    -> Route (mask, row_cnt, row_idx, head_cnt)
    schedule(problem, row_cnt)           -> work list (longest first)
    augment(problem, route, worker_of, worker_load, ws) -> slack-aware augmentation, in place
    sparse_fwd(q, k, v, route, ..., causal) -> (o, lse)
    dense_fwd(q, k, v, block, causal)    -> (o, lse)
and a convenience ``sparse_attention`` that runs all three sparse steps.
``causal=True`` routes each query block over key blocks j <= i only and masks
keys after each query token.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattn_tbs.so")

ATTN_OK, ATTN_E_INVALID, ATTN_E_UNSUPPORTED, ATTN_E_WORKSPACE, ATTN_E_DEVICE = 0, 1, 2, 3, 4
ATTN_DTYPE_BF16, ATTN_DTYPE_F32 = 0, 1
OP_ROUTE, OP_SCHEDULE, OP_SPARSE_FWD, OP_DENSE_FWD, OP_AUGMENT = 0, 1, 2, 3, 4
FLAG_PROFILE_WORKERS = 1
FLAG_NO_SPLIT = 2        # run every work item whole (no split along the keys)
CTRL_BYTES = 256
DEFAULT_HEAD_WINDOW = 4
# Head windows keep the K/V of the heads that run together cache-resident;
# past this many K+V bytes per head they no longer fit and only cost balance.
HEAD_WINDOW_MAX_KV_BYTES = 32 << 20


def default_head_window(problem: "Problem") -> int:
    """Heads per scheduling window used when none is given: DEFAULT_HEAD_WINDOW
    while one head's K and V fit in HEAD_WINDOW_MAX_KV_BYTES, else 0 (a single
    longest-first list over all heads)."""
    elem = 2 if problem.dtype == ATTN_DTYPE_BF16 else 4
    kv = 2 * problem.seq_len * problem.head_dim * elem
    return DEFAULT_HEAD_WINDOW if kv <= HEAD_WINDOW_MAX_KV_BYTES else 0

_STATUS_NAMES = {1: "ATTN_E_INVALID", 2: "ATTN_E_UNSUPPORTED", 3: "ATTN_E_WORKSPACE", 4: "ATTN_E_DEVICE"}


class AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("seq_len", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("flags", ctypes.c_int32),
        ("scale", ctypes.c_double),
        ("key_block", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]

    @property
    def num_blocks(self) -> int:
        """Query blocks per sequence, nb."""
        return -(-self.seq_len // self.block)

    @property
    def kblock(self) -> int:
        return self.key_block or self.block

    @property
    def num_key_blocks(self) -> int:
        """Key blocks per sequence, nbk (entries per row of the routing outputs)."""
        return -(-self.seq_len // self.kblock)

    @property
    def units(self) -> int:
        return self.batch * self.heads * self.num_blocks

    @property
    def group(self) -> int:
        """Query blocks per work item of the fwd kernel (attn_group_size)."""
        g = int(lib().attn_group_size(ctypes.byref(self)))
        if g == 0:
            _check(ATTN_E_INVALID)
        return g

    @property
    def items(self) -> int:
        g = self.group
        return self.batch * self.heads * (-(-self.num_blocks // g))


_lib = None


def lib() -> ctypes.CDLL:
    """Load libattn_tbs.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                           "(run `python -c 'import __graft_entry__ as g; g.build()'`)")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(Problem)
    vp, i32, sz, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_double
    L.attn_abi_version.restype = i32
    L.attn_abi_version.argtypes = []
    L.attn_last_error.restype = ctypes.c_char_p
    L.attn_last_error.argtypes = []
    L.attn_workspace_bytes.restype = sz
    L.attn_workspace_bytes.argtypes = [P, i32]
    L.attn_group_size.restype = i32
    L.attn_group_size.argtypes = [P]
    L.attn_num_workers.restype = i32
    L.attn_num_workers.argtypes = [P, i32]
    L.attn_route.restype = i32
    L.attn_route.argtypes = [P, vp, vp, dbl, vp, vp, vp, vp, vp, vp, sz, vp]
    L.attn_schedule.restype = i32
    L.attn_schedule.argtypes = [P, vp, i32, i32, vp, vp, vp, vp, sz, vp]
    L.attn_sparse_fwd.restype = i32
    L.attn_sparse_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.attn_sparse_fwd_noalloc.restype = i32
    L.attn_sparse_fwd_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.attn_dense_fwd.restype = i32
    L.attn_dense_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, sz, vp]
    L.attn_augment.restype = i32
    L.attn_augment.argtypes = [P, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.attn_augment_union.restype = i32
    L.attn_augment_union.argtypes = [P, vp, vp, vp, vp, vp]
    L.attn_quantize_qk_fp8.restype = i32
    L.attn_quantize_qk_fp8.argtypes = [P, vp, vp, vp, vp, vp, vp, vp]
    L.attn_route_fp8.restype = i32
    L.attn_route_fp8.argtypes = [P, vp, vp, dbl, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.attn_sparse_fwd_fp8.restype = i32
    L.attn_sparse_fwd_fp8.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.attn_dense_fwd_fp8.restype = i32
    L.attn_dense_fwd_fp8.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    _lib = L
    return L


def _check(status: int):
    if status != ATTN_OK:
        raise AttnError(status, lib().attn_last_error().decode(errors="replace"))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return ATTN_DTYPE_BF16
    if dt == torch.float32:
        return ATTN_DTYPE_F32
    raise ValueError(f"unsupported dtype {dt} (bfloat16 or float32)")


def _require_device(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must live in GPU memory")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def make_problem(q: torch.Tensor, block: int, causal: bool = False, scale: Optional[float] = None,
                 flags: int = 0, key_block: Optional[int] = None) -> Problem:
    if q.dim() != 4:
        raise ValueError(f"q must be [B, H, N, d], got shape {tuple(q.shape)}")
    B, H, N, d = q.shape
    return Problem(B, H, N, d, block, _dtype_code(q.dtype), int(bool(causal)), flags,
                   0.0 if scale is None else float(scale), int(key_block or 0), 0)


def workspace_bytes(problem: Problem, op: Optional[int] = None) -> int:
    ops = [op] if op is not None else [OP_ROUTE, OP_SCHEDULE, OP_SPARSE_FWD, OP_DENSE_FWD, OP_AUGMENT]
    n = max(lib().attn_workspace_bytes(ctypes.byref(problem), o) for o in ops)
    if n == 0:
        _check(ATTN_E_INVALID)
    return n


def workspace(problem: Problem, device=None, op: Optional[int] = None) -> torch.Tensor:
    """A zero-filled workspace large enough for `op` (default: every op)."""
    return torch.zeros(workspace_bytes(problem, op), dtype=torch.uint8, device=device or "cuda")


def num_workers(problem: Problem, op: int = OP_SPARSE_FWD) -> int:
    return int(lib().attn_num_workers(ctypes.byref(problem), op))


_num_workers = num_workers     # for functions whose num_workers argument hides it


@dataclasses.dataclass
class Route:
    problem: Problem
    top_p: float
    mask: torch.Tensor       # [B,H,nb,nbk] uint8
    row_cnt: torch.Tensor    # [B,H,nb] int32
    row_idx: torch.Tensor    # [B,H,nb,nbk] int32 (selected prefix of row_cnt entries, then the ranked tail)
    head_cnt: torch.Tensor   # [B,H] int32
    block_prob: Optional[torch.Tensor] = None   # [B,H,nb,nbk] float64


def route(q: torch.Tensor, k: torch.Tensor, top_p: float, block: int, scale: Optional[float] = None,
          ws: Optional[torch.Tensor] = None, return_prob: bool = False, out: Optional[Route] = None,
          causal: bool = False, key_block: Optional[int] = None) -> Route:
    """attn_route: block pooling, scores, softmax and top-p cut (all on the GPU)."""
    _require_device(q, k)
    if k.shape != q.shape or k.dtype != q.dtype:
        raise ValueError("q and k must share shape and dtype")
    pr = make_problem(q, block, causal=causal, scale=scale, key_block=key_block)
    B, H, nb, nbk = pr.batch, pr.heads, pr.num_blocks, pr.num_key_blocks
    dev = q.device
    if out is None:
        out = Route(pr, float(top_p),
                    torch.empty((B, H, nb, nbk), dtype=torch.uint8, device=dev),
                    torch.empty((B, H, nb), dtype=torch.int32, device=dev),
                    torch.empty((B, H, nb, nbk), dtype=torch.int32, device=dev),
                    torch.empty((B, H), dtype=torch.int32, device=dev),
                    torch.empty((B, H, nb, nbk), dtype=torch.float64, device=dev) if return_prob else None)
    out.problem, out.top_p = pr, float(top_p)
    if ws is None:
        ws = workspace(pr, dev, OP_ROUTE)
    _check(lib().attn_route(ctypes.byref(pr), _ptr(q), _ptr(k), float(top_p), _ptr(out.mask), _ptr(out.row_cnt),
                            _ptr(out.row_idx), _ptr(out.head_cnt), _ptr(out.block_prob), _ptr(ws),
                            ws.numel(), _stream()))
    return out


def schedule(problem: Problem, row_cnt: torch.Tensor, ws: torch.Tensor, head_window: Optional[int] = None,
             num_workers: int = 0, lpt: bool = False, work_list: Optional[torch.Tensor] = None,
             worker_of: Optional[torch.Tensor] = None, worker_load: Optional[torch.Tensor] = None):
    """attn_schedule: longest-first work list inside windows of `head_window`
    heads (0: one window; None: default_head_window(problem)); with lpt=True
    also the greedy LPT assignment (worker_of, worker_load), for load-balance
    reports and augment()."""
    _require_device(row_cnt, ws)
    if head_window is None:
        head_window = default_head_window(problem)
    dev = row_cnt.device
    n_items = problem.items
    if work_list is None:
        work_list = torch.empty(n_items, dtype=torch.int32, device=dev)
    if lpt:
        W = num_workers or torch.cuda.get_device_properties(dev).multi_processor_count
        if worker_of is None:
            worker_of = torch.empty(n_items, dtype=torch.int32, device=dev)
        if worker_load is None:
            worker_load = torch.empty(W, dtype=torch.int64, device=dev)
        num_workers = worker_load.numel()
    else:
        worker_of = worker_load = None
    _check(lib().attn_schedule(ctypes.byref(problem), _ptr(row_cnt), int(head_window), int(num_workers),
                               _ptr(work_list),
                               _ptr(worker_of), _ptr(worker_load), _ptr(ws), ws.numel(), _stream()))
    if lpt:
        return work_list, worker_of, worker_load
    return work_list


SASA_TILE_FIXED = 3        # ATTN_SASA_TILE_FIXED: fixed cost of a tile, in row-tiles


@dataclasses.dataclass
class Augmentation:
    worker_of: torch.Tensor     # [items] int32, the worker of every work item
    worker_load: torch.Tensor   # [W] int64, cost per worker (row-tiles) before augmentation
    paid: torch.Tensor          # [W] int32, (row, block) pairs bought per worker


def augment(problem: Problem, r: Route, ws: torch.Tensor, work_list: Optional[torch.Tensor] = None,
            num_workers: int = 0, out: Optional[Augmentation] = None) -> Augmentation:
    """attn_augment: slack-aware augmentation of the routing `r` in place,
    priced in row-tiles (items assigned in batches of W work-list positions,
    each worker buying (row, block) pairs for its last item with its slack).
    r needs its block probabilities (route(..., return_prob=True)); work_list
    from schedule() over the same routing (None: item order); num_workers 0 =
    the fwd kernel's workgroups."""
    if r.block_prob is None:
        raise ValueError("augment needs the block probabilities: route(..., return_prob=True)")
    _require_device(ws, r.mask, r.row_cnt, r.row_idx, r.head_cnt, r.block_prob, work_list)
    dev = r.row_cnt.device
    if out is None:
        W = num_workers or _num_workers(problem, OP_SPARSE_FWD)
        out = Augmentation(torch.empty(problem.items, dtype=torch.int32, device=dev),
                           torch.empty(W, dtype=torch.int64, device=dev),
                           torch.empty(W, dtype=torch.int32, device=dev))
    W = out.worker_load.numel()
    _check(lib().attn_augment(ctypes.byref(problem), _ptr(r.block_prob), _ptr(work_list), int(W), _ptr(r.mask),
                              _ptr(r.row_cnt), _ptr(r.row_idx), _ptr(r.head_cnt), _ptr(out.worker_of),
                              _ptr(out.worker_load), _ptr(out.paid), _ptr(ws), ws.numel(), _stream()))
    return out


def augment_union(problem: Problem, r: Route) -> Route:
    """attn_augment_union: every row takes the eligible blocks of its work
    item's union (the idle wave-steps inside the item), in place."""
    _require_device(r.mask, r.row_cnt, r.row_idx, r.head_cnt)
    _check(lib().attn_augment_union(ctypes.byref(problem), _ptr(r.mask), _ptr(r.row_cnt), _ptr(r.row_idx),
                                    _ptr(r.head_cnt), _stream()))
    return r


def _out_tensors(q, o, lse, want_lse):
    B, H, N, d = q.shape
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    return o, lse


def sparse_fwd(q, k, v, row_cnt, row_idx, block: int, work_list=None, scale: Optional[float] = None,
               ws: Optional[torch.Tensor] = None, o=None, lse=None, want_lse: bool = True, flags: int = 0,
               causal: bool = False, key_block: Optional[int] = None):
    """attn_sparse_fwd: attention of each query block over its selected key blocks."""
    _require_device(q, k, v, row_cnt, row_idx, work_list)
    pr = make_problem(q, block, causal=causal, scale=scale, flags=flags, key_block=key_block)
    o, lse = _out_tensors(q, o, lse, want_lse)
    if ws is None:
        ws = workspace(pr, q.device, OP_SPARSE_FWD)
    _check(lib().attn_sparse_fwd(ctypes.byref(pr), _ptr(q), _ptr(k), _ptr(v), _ptr(row_cnt), _ptr(row_idx),
                                 _ptr(work_list), _ptr(o), _ptr(lse), _ptr(ws), ws.numel(), _stream()))
    return o, lse


def sparse_fwd_noalloc(q, k, v, row_cnt, row_idx, block: int, work_list=None, scale: Optional[float] = None,
                       o=None, lse=None, want_lse: bool = True, flags: int = 0, causal: bool = False,
                       key_block: Optional[int] = None):
    """attn_sparse_fwd_noalloc: attn_sparse_fwd whose queue counters live in the
    library's static per-GPU scratch (no workspace).  Pass o (and lse) to keep
    the call free of allocations; calls on one GPU must not overlap."""
    _require_device(q, k, v, row_cnt, row_idx, work_list)
    pr = make_problem(q, block, causal=causal, scale=scale, flags=flags, key_block=key_block)
    o, lse = _out_tensors(q, o, lse, want_lse)
    _check(lib().attn_sparse_fwd_noalloc(ctypes.byref(pr), _ptr(q), _ptr(k), _ptr(v), _ptr(row_cnt),
                                         _ptr(row_idx), _ptr(work_list), _ptr(o), _ptr(lse), _stream()))
    return o, lse


def dense_fwd(q, k, v, block: int, causal: bool = False, scale: Optional[float] = None,
              ws: Optional[torch.Tensor] = None, o=None, lse=None, want_lse: bool = True, flags: int = 0):
    """attn_dense_fwd: dense (optionally causal) attention, the p = 1 case."""
    _require_device(q, k, v)
    pr = make_problem(q, block, causal=causal, scale=scale, flags=flags)
    o, lse = _out_tensors(q, o, lse, want_lse)
    if ws is None:
        ws = workspace(pr, q.device, OP_DENSE_FWD)
    _check(lib().attn_dense_fwd(ctypes.byref(pr), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(ws),
                                ws.numel(), _stream()))
    return o, lse


FP8_TILE = 64   # keys per K scale of the fp8 path


@dataclasses.dataclass
class QuantizedQK:
    q8: torch.Tensor        # [B,H,N,d] uint8 E4M3 codes
    q_scale: torch.Tensor   # [B,H,N] float32, one per token
    k8: torch.Tensor        # [B,H,N,d] uint8 E4M3 codes
    k_scale: torch.Tensor   # [B,H,ceil(N/64)] float32, one per 64-token tile


def quantize_qk_fp8(q: torch.Tensor, k: torch.Tensor, block: int = 64, out: Optional[QuantizedQK] = None,
                    key_block: Optional[int] = None) -> QuantizedQK:
    """attn_quantize_qk_fp8: E4M3 codes of Q (scale per token) and K (scale per 64-token tile)."""
    _require_device(q, k)
    if k.shape != q.shape or k.dtype != q.dtype:
        raise ValueError("q and k must share shape and dtype")
    pr = make_problem(q, block, key_block=key_block)
    B, H, N, d = q.shape
    if out is None:
        dev = q.device
        out = QuantizedQK(torch.empty((B, H, N, d), dtype=torch.uint8, device=dev),
                          torch.empty((B, H, N), dtype=torch.float32, device=dev),
                          torch.empty((B, H, N, d), dtype=torch.uint8, device=dev),
                          torch.empty((B, H, -(-N // FP8_TILE)), dtype=torch.float32, device=dev))
    _check(lib().attn_quantize_qk_fp8(ctypes.byref(pr), _ptr(q), _ptr(k), _ptr(out.q8), _ptr(out.q_scale),
                                      _ptr(out.k8), _ptr(out.k_scale), _stream()))
    return out


def _new_quantized(q: torch.Tensor) -> QuantizedQK:
    B, H, N, d = q.shape
    dev = q.device
    return QuantizedQK(torch.empty((B, H, N, d), dtype=torch.uint8, device=dev),
                       torch.empty((B, H, N), dtype=torch.float32, device=dev),
                       torch.empty((B, H, N, d), dtype=torch.uint8, device=dev),
                       torch.empty((B, H, -(-N // FP8_TILE)), dtype=torch.float32, device=dev))


def route_fp8(q: torch.Tensor, k: torch.Tensor, top_p: float, block: int, scale: Optional[float] = None,
              ws: Optional[torch.Tensor] = None, return_prob: bool = False, out: Optional[Route] = None,
              qk_out: Optional[QuantizedQK] = None, causal: bool = False, key_block: Optional[int] = None):
    """attn_route_fp8: attn_route and attn_quantize_qk_fp8 in one read of Q and K.
    Returns (Route, QuantizedQK)."""
    _require_device(q, k)
    if k.shape != q.shape or k.dtype != q.dtype:
        raise ValueError("q and k must share shape and dtype")
    pr = make_problem(q, block, causal=causal, scale=scale, key_block=key_block)
    B, H, nb, nbk = pr.batch, pr.heads, pr.num_blocks, pr.num_key_blocks
    dev = q.device
    if out is None:
        out = Route(pr, float(top_p),
                    torch.empty((B, H, nb, nbk), dtype=torch.uint8, device=dev),
                    torch.empty((B, H, nb), dtype=torch.int32, device=dev),
                    torch.empty((B, H, nb, nbk), dtype=torch.int32, device=dev),
                    torch.empty((B, H), dtype=torch.int32, device=dev),
                    torch.empty((B, H, nb, nbk), dtype=torch.float64, device=dev) if return_prob else None)
    out.problem, out.top_p = pr, float(top_p)
    if qk_out is None:
        qk_out = _new_quantized(q)
    if ws is None:
        ws = workspace(pr, dev, OP_ROUTE)
    _check(lib().attn_route_fp8(ctypes.byref(pr), _ptr(q), _ptr(k), float(top_p), _ptr(out.mask), _ptr(out.row_cnt),
                                _ptr(out.row_idx), _ptr(out.head_cnt), _ptr(out.block_prob), _ptr(qk_out.q8),
                                _ptr(qk_out.q_scale), _ptr(qk_out.k8), _ptr(qk_out.k_scale), _ptr(ws), ws.numel(),
                                _stream()))
    return out, qk_out


def _fp8_problem(qk: QuantizedQK, v: torch.Tensor, block: int, causal: bool, scale, flags, key_block):
    _require_device(qk.q8, qk.q_scale, qk.k8, qk.k_scale, v)
    if qk.q8.shape != v.shape or qk.k8.shape != v.shape:
        raise ValueError("q8, k8 and v must share the shape [B, H, N, d]")
    return make_problem(v, block, causal=causal, scale=scale, flags=flags, key_block=key_block)


def sparse_fwd_fp8(qk: QuantizedQK, v, row_cnt, row_idx, block: int, work_list=None,
                   scale: Optional[float] = None, ws: Optional[torch.Tensor] = None, o=None, lse=None,
                   want_lse: bool = True, flags: int = 0, causal: bool = False, key_block: Optional[int] = None):
    """attn_sparse_fwd_fp8: sparse_fwd with E4M3 Q and K (S = Q K^T on fp8 MFMA)."""
    _require_device(row_cnt, row_idx, work_list)
    pr = _fp8_problem(qk, v, block, causal, scale, flags, key_block)
    o, lse = _out_tensors(v, o, lse, want_lse)
    if ws is None:
        ws = workspace(pr, v.device, OP_SPARSE_FWD)
    _check(lib().attn_sparse_fwd_fp8(ctypes.byref(pr), _ptr(qk.q8), _ptr(qk.q_scale), _ptr(qk.k8), _ptr(qk.k_scale),
                                     _ptr(v), _ptr(row_cnt), _ptr(row_idx), _ptr(work_list), _ptr(o), _ptr(lse),
                                     _ptr(ws), ws.numel(), _stream()))
    return o, lse


def dense_fwd_fp8(qk: QuantizedQK, v, block: int, causal: bool = False, scale: Optional[float] = None,
                  ws: Optional[torch.Tensor] = None, o=None, lse=None, want_lse: bool = True, flags: int = 0):
    """attn_dense_fwd_fp8: dense (optionally causal) attention with E4M3 Q and K."""
    pr = _fp8_problem(qk, v, block, causal, scale, flags, None)
    o, lse = _out_tensors(v, o, lse, want_lse)
    if ws is None:
        ws = workspace(pr, v.device, OP_DENSE_FWD)
    _check(lib().attn_dense_fwd_fp8(ctypes.byref(pr), _ptr(qk.q8), _ptr(qk.q_scale), _ptr(qk.k8), _ptr(qk.k_scale),
                                    _ptr(v), _ptr(o), _ptr(lse), _ptr(ws), ws.numel(), _stream()))
    return o, lse


def sparse_attention(q, k, v, top_p: float, block: int, scale: Optional[float] = None,
                     ws: Optional[torch.Tensor] = None, want_lse: bool = True,
                     head_window: Optional[int] = None, causal: bool = False, sasa: bool = False,
                     num_workers: int = 0, key_block: Optional[int] = None, fp8: bool = False):
    """route -> schedule -> sparse_fwd on the current stream; returns (o, lse, route, work_list).

    With sasa=True: route -> schedule -> augment (priced in union tiles over
    that work list) -> sparse_fwd on the same work list, so the kernel takes
    the items in the order the augmentation's assignment assumed.  With
    fp8=True the routing
    pass also quantises Q and K to E4M3 (route_fp8: one read of Q and K) and the
    forward is sparse_fwd_fp8; routing reads the bf16 Q and K either way."""
    pr = make_problem(q, block, causal=causal, scale=scale, key_block=key_block)
    if ws is None:
        ws = workspace(pr, q.device)
    if fp8:
        r, qk = route_fp8(q, k, top_p, block, scale=scale, ws=ws, causal=causal, return_prob=sasa,
                          key_block=key_block)
    else:
        r = route(q, k, top_p, block, scale=scale, ws=ws, causal=causal, return_prob=sasa, key_block=key_block)
    wl = schedule(pr, r.row_cnt, ws, head_window=head_window)
    if sasa:
        augment(pr, r, ws, work_list=wl, num_workers=num_workers)
    if fp8:
        o, lse = sparse_fwd_fp8(qk, v, r.row_cnt, r.row_idx, block, work_list=wl, scale=scale, ws=ws,
                                want_lse=want_lse, causal=causal, key_block=key_block)
    else:
        o, lse = sparse_fwd(q, k, v, r.row_cnt, r.row_idx, block, work_list=wl, scale=scale, ws=ws,
                            want_lse=want_lse, causal=causal, key_block=key_block)
    return o, lse, r, wl


__all__ = [
    "lib", "AttnError", "Problem", "Route", "make_problem", "default_head_window", "workspace", "workspace_bytes", "num_workers",
    "route", "schedule", "augment", "Augmentation", "SASA_TILE_FIXED", "augment_union", "sparse_fwd", "sparse_fwd_noalloc", "dense_fwd",
    "sparse_attention", "LIB_PATH",
    "QuantizedQK", "quantize_qk_fp8", "route_fp8", "sparse_fwd_fp8", "dense_fwd_fp8", "FP8_TILE",
]
