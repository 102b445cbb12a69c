"""The C ABI without a GPU: the library loads, exports every symbol the header
declares, reports sizes, and rejects bad arguments with the documented
status codes before any HIP call is made (no compute runs here)."""
import ctypes
import math
import os
import re

import pytest

import top_block_sparse_pool_amd as tbs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_tbs.h")

pytestmark = pytest.mark.skipif(not os.path.exists(tbs.LIB_PATH), reason="HIP library not built")

FAKE = ctypes.c_void_p(0x10000)       # aligned, never dereferenced: validation fails first
WS = ctypes.c_void_p(0x20000)


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\S.*?\b(attn_[a-z0-9_]+)\(", text, flags=re.M)))


def test_exports_every_declared_symbol():
    L = tbs.lib()
    names = _declared_functions()
    assert set(names) == {"attn_abi_version", "attn_last_error", "attn_workspace_bytes", "attn_num_workers",
                          "attn_group_size", "attn_route", "attn_schedule", "attn_augment", "attn_augment_union",
                          "attn_sparse_fwd", "attn_sparse_fwd_noalloc", "attn_dense_fwd", "attn_quantize_qk_fp8",
                          "attn_route_fp8", "attn_sparse_fwd_fp8", "attn_dense_fwd_fp8"}
    for n in names:
        assert hasattr(L, n), n
    assert L.attn_abi_version() == 8


def _problem(B=1, H=40, N=32760, d=128, block=64, dtype=0, causal=0, flags=0, scale=0.0, key_block=0, reserved=0):
    return tbs.Problem(B, H, N, d, block, dtype, causal, flags, scale, key_block, reserved)


def test_struct_layout_matches_header():
    assert ctypes.sizeof(tbs.Problem) == 48
    assert tbs.Problem.scale.offset == 32
    assert tbs.Problem.key_block.offset == 40 and tbs.Problem.reserved.offset == 44


def test_group_size():
    L = tbs.lib()
    # bf16: 256 query rows per work item; fp32: one block
    assert L.attn_group_size(ctypes.byref(_problem())) == 4
    assert L.attn_group_size(ctypes.byref(_problem(block=128))) == 2
    assert L.attn_group_size(ctypes.byref(_problem(dtype=1))) == 1
    assert L.attn_group_size(ctypes.byref(_problem(d=80))) == 0
    assert _problem(N=1000).items == 40 * 4


def test_workspace_sizes():
    L = tbs.lib()
    p = _problem()
    nb = 512
    assert L.attn_workspace_bytes(ctypes.byref(p), tbs.OP_ROUTE) == 256 + 2 * 8 * 40 * nb * 128
    pk = _problem(block=128, key_block=64)
    assert L.attn_workspace_bytes(ctypes.byref(pk), tbs.OP_ROUTE) == 256 + 8 * 40 * (256 + 512) * 128
    assert L.attn_workspace_bytes(ctypes.byref(p), tbs.OP_SCHEDULE) == 256
    assert L.attn_workspace_bytes(ctypes.byref(p), tbs.OP_SPARSE_FWD) == 256
    p.flags = tbs.FLAG_PROFILE_WORKERS
    assert L.attn_workspace_bytes(ctypes.byref(p), tbs.OP_DENSE_FWD) == 256 + 16 * 4096
    U = 40 * nb
    up = lambda x: (x + 255) // 256 * 256
    items, W = U // 4, 4096
    # item bitmaps (16 words), item tiles, item costs, last items, bought
    # pairs (4 rows x 32 words per worker), worker of every item, loads,
    # pairs bought, makespan
    assert L.attn_workspace_bytes(ctypes.byref(p), tbs.OP_AUGMENT) == (
        256 + up(items * 16 * 4) + 2 * up(items * 4) + up(W * 4) + up(W * 4 * 32 * 4) + up(items * 4) + up(W * 8)
        + up(W * 4) + 256)
    assert L.attn_workspace_bytes(ctypes.byref(p), 9) == 0
    assert L.attn_workspace_bytes(None, 0) == 0


def _route(p, top_p=0.9, q=FAKE, k=FAKE, ws=WS, ws_bytes=1 << 40, mask=FAKE, rc=FAKE, ri=FAKE, hc=FAKE):
    return tbs.lib().attn_route(ctypes.byref(p) if p is not None else None, q, k, top_p, mask, rc, ri, hc,
                                None, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), 1), (dict(H=-1), 1), (dict(N=0), 1), (dict(d=96), 2), (dict(d=0), 1), (dict(block=32), 2),
    (dict(dtype=7), 1), (dict(causal=2), 1), (dict(flags=8), 1), (dict(scale=-1.0), 1),
    (dict(scale=math.inf), 1), (dict(N=64 * 1025), 2), (dict(key_block=96), 2), (dict(key_block=-64), 1),
    (dict(reserved=1), 1), (dict(block=128, key_block=64, N=64 * 1025), 2),
])
def test_route_rejects_bad_problem(kw, code):
    assert _route(_problem(**kw)) == code
    assert tbs.lib().attn_last_error().decode() != ""


@pytest.mark.parametrize("top_p", [0.0, -0.5, 1.5, math.nan])
def test_route_rejects_bad_top_p(top_p):
    assert _route(_problem(), top_p=top_p) == 1


def test_route_rejects_pointers_and_workspace():
    p = _problem()
    assert _route(None) == 1
    assert _route(p, q=None) == 1
    assert _route(p, k=ctypes.c_void_p(0x10008)) == 1        # not 16-byte aligned
    assert _route(p, mask=None) == 1
    assert _route(p, rc=ctypes.c_void_p(0x10002)) == 1
    assert _route(p, ws=None) == 3
    assert _route(p, ws_bytes=1000) == 3
    assert _route(p, ws=ctypes.c_void_p(0x20008)) == 3
    assert "workspace" in tbs.lib().attn_last_error().decode()


def test_schedule_and_fwd_validation():
    L = tbs.lib()
    p = _problem()
    assert L.attn_schedule(ctypes.byref(p), FAKE, 4, -1, FAKE, None, None, WS, 1 << 20, None) == 1
    assert L.attn_schedule(ctypes.byref(p), FAKE, 4, 5000, FAKE, None, None, WS, 1 << 20, None) == 1
    assert L.attn_schedule(ctypes.byref(p), FAKE, -1, 0, FAKE, None, None, WS, 1 << 20, None) == 1
    assert L.attn_schedule(ctypes.byref(p), None, 4, 0, FAKE, None, None, WS, 1 << 20, None) == 1
    assert L.attn_schedule(ctypes.byref(p), FAKE, 4, 0, FAKE, None, None, WS, 100, None) == 3
    assert L.attn_sparse_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, None, FAKE, None, FAKE, None, WS, 1 << 20,
                             None) == 1
    assert L.attn_sparse_fwd(ctypes.byref(p), FAKE, FAKE, ctypes.c_void_p(0x10004), FAKE, FAKE, None, FAKE,
                             None, WS, 1 << 20, None) == 1
    assert L.attn_sparse_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, WS, 16, None) == 3
    big = _problem(N=64 * 2049)
    assert L.attn_sparse_fwd(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, WS, 1 << 20,
                             None) == 2
    pc = _problem(causal=1)                       # causal is accepted; argument checks still apply
    assert L.attn_sparse_fwd(ctypes.byref(pc), FAKE, FAKE, FAKE, None, FAKE, None, FAKE, None, WS, 1 << 20,
                             None) == 1
    assert _route(_problem(causal=1), top_p=0.0) == 1
    assert _route(_problem(causal=1, N=64 * 1025)) == 2
    assert L.attn_dense_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, None, None, WS, 1 << 20, None) == 1
    assert L.attn_dense_fwd(ctypes.byref(_problem(d=80)), FAKE, FAKE, FAKE, FAKE, None, WS, 1 << 20, None) == 2
    assert L.attn_dense_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, ctypes.c_void_p(0x10001), WS, 1 << 20,
                            None) == 1


def test_augment_validation():
    L = tbs.lib()
    p = _problem()
    D = ctypes.c_void_p(0x10000)

    def aug(pr=p, bp=D, wlist=D, W=256, mask=D, rc=D, ri=D, hc=D, wo=None, wl=None, paid=None, ws=WS, wsb=1 << 30):
        return L.attn_augment(ctypes.byref(pr) if pr is not None else None, bp, wlist, W, mask, rc, ri, hc, wo, wl,
                              paid, ws, wsb, None)
    assert aug(pr=None) == 1
    assert aug(W=0) == 1 and aug(W=4097) == 1
    assert aug(bp=None) == 1 and aug(bp=ctypes.c_void_p(0x10004)) == 1
    assert aug(wl=ctypes.c_void_p(0x10004)) == 1 and aug(wlist=ctypes.c_void_p(0x10002)) == 1
    assert aug(mask=None) == 1 and aug(rc=None) == 1 and aug(ri=ctypes.c_void_p(0x10002)) == 1
    assert aug(paid=ctypes.c_void_p(0x10001)) == 1 and aug(wo=ctypes.c_void_p(0x10001)) == 1
    assert aug(pr=_problem(N=64 * 1025)) == 2
    assert aug(wsb=1000) == 3 and aug(ws=None) == 3
    assert "workspace" in L.attn_last_error().decode()


def test_augment_union_validation():
    L = tbs.lib()
    D = ctypes.c_void_p(0x10000)
    p = _problem()
    assert L.attn_augment_union(None, D, D, D, D, None) == 1
    assert L.attn_augment_union(ctypes.byref(p), None, D, D, D, None) == 1
    assert L.attn_augment_union(ctypes.byref(p), D, ctypes.c_void_p(0x10002), D, D, None) == 1
    assert L.attn_augment_union(ctypes.byref(p), D, D, D, None, None) == 1
    assert L.attn_augment_union(ctypes.byref(_problem(N=64 * 1025)), D, D, D, D, None) == 2


def test_fp8_validation():
    L = tbs.lib()
    D = ctypes.c_void_p(0x10000)
    p = _problem()

    def quant(pr=p, q=D, k=D, q8=D, qs=D, k8=D, ks=D):
        return L.attn_quantize_qk_fp8(ctypes.byref(pr) if pr is not None else None, q, k, q8, qs, k8, ks, None)
    assert quant(pr=None) == 1
    assert quant(pr=_problem(d=64)) == 2 and "head_dim" in L.attn_last_error().decode()
    assert quant(pr=_problem(dtype=1)) == 2
    assert quant(q=None) == 1 and quant(k8=ctypes.c_void_p(0x10008)) == 1
    assert quant(qs=None) == 1 and quant(ks=ctypes.c_void_p(0x10002)) == 1

    def sfwd(pr=p, q8=D, qs=D, k8=D, ks=D, v=D, rc=D, ri=D, wl=None, o=D, lse=None, ws=WS, wsb=1 << 20):
        return L.attn_sparse_fwd_fp8(ctypes.byref(pr), q8, qs, k8, ks, v, rc, ri, wl, o, lse, ws, wsb, None)
    assert sfwd(pr=_problem(d=64)) == 2 and sfwd(pr=_problem(dtype=1)) == 2
    assert sfwd(qs=None) == 1 and sfwd(ks=None) == 1 and sfwd(q8=ctypes.c_void_p(0x10004)) == 1
    assert sfwd(rc=None) == 1 and sfwd(ri=ctypes.c_void_p(0x10002)) == 1 and sfwd(v=None) == 1
    assert sfwd(wsb=16) == 3
    assert sfwd(pr=_problem(N=64 * 2049)) == 2

    def dfwd(pr=p, q8=D, qs=D, k8=D, ks=D, v=D, o=D, lse=None, ws=WS, wsb=1 << 20):
        return L.attn_dense_fwd_fp8(ctypes.byref(pr), q8, qs, k8, ks, v, o, lse, ws, wsb, None)
    assert dfwd(pr=_problem(d=64)) == 2 and dfwd(qs=None) == 1 and dfwd(o=None) == 1
    assert dfwd(lse=ctypes.c_void_p(0x10001)) == 1 and dfwd(ws=None) == 3


def test_sparse_fwd_noalloc_validation():
    # Bad arguments and a problem whose workspace exceeds the static scratch
    # (the worker-profiling flag) are rejected before any HIP call.
    L = tbs.lib()
    pr = _problem(N=4096, H=2)
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None]
    st = L.attn_sparse_fwd_noalloc(ctypes.byref(_problem(N=4096, H=2, flags=tbs.FLAG_PROFILE_WORKERS)), *args)
    assert st == tbs.ATTN_E_WORKSPACE
    assert b"static array holds 256" in L.attn_last_error()
    st = L.attn_sparse_fwd_noalloc(ctypes.byref(pr), None, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None)
    assert st == tbs.ATTN_E_INVALID and b"q is NULL" in L.attn_last_error()
    st = L.attn_sparse_fwd_noalloc(ctypes.byref(pr), FAKE, FAKE, FAKE, None, FAKE, None, FAKE, FAKE, None)
    assert st == tbs.ATTN_E_INVALID and b"row_cnt" in L.attn_last_error()
    st = L.attn_sparse_fwd_noalloc(ctypes.byref(pr), FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                   ctypes.c_void_p(0x10004), FAKE, None)
    assert st == tbs.ATTN_E_INVALID and b"o is not 16-byte aligned" in L.attn_last_error()
    st = L.attn_sparse_fwd_noalloc(ctypes.byref(_problem(d=80)), *args)
    assert st == tbs.ATTN_E_UNSUPPORTED


def test_route_fp8_validation():
    L = tbs.lib()
    args = [FAKE, FAKE, ctypes.c_double(0.9), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, WS,
            ctypes.c_size_t(1 << 30), None]
    assert L.attn_route_fp8(ctypes.byref(_problem(d=64)), *args) == tbs.ATTN_E_UNSUPPORTED
    assert L.attn_route_fp8(ctypes.byref(_problem(dtype=1)), *args) == tbs.ATTN_E_UNSUPPORTED
    bad = list(args)
    bad[8] = None                                                     # q8
    assert L.attn_route_fp8(ctypes.byref(_problem(N=4096)), *bad) == tbs.ATTN_E_INVALID
    assert b"q8" in L.attn_last_error()
    bad = list(args)
    bad[2] = ctypes.c_double(1.5)                                     # top_p
    assert L.attn_route_fp8(ctypes.byref(_problem(N=4096)), *bad) == tbs.ATTN_E_INVALID
    small = list(args)
    small[13] = ctypes.c_size_t(64)                                   # workspace too small
    assert L.attn_route_fp8(ctypes.byref(_problem(N=4096)), *small) == tbs.ATTN_E_WORKSPACE
