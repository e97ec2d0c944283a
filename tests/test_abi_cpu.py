"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every
symbol the header declares, reports its version and status strings, sizes its
workspaces, and rejects bad arguments before anything is enqueued.

Only argument errors are exercised here: every call below fails validation on
the host, so no kernel is launched and no device memory is touched (the
pointers are dummies)."""
import ctypes
import os
import re

import pytest

import nvfp4_moe_expert_amd as nv

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "nvfp4.h")
A = 0x100000          # 16-byte aligned dummy device address
B = 0x200000
OK, ENULL, ESHAPE, EALIGN, EWS, EUNSUP, ESCRATCH = 0, 1, 2, 3, 4, 5, 7


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_[a-z0-9_]+)\s*\(", text)))


def test_library_is_built_and_loads():
    assert os.path.exists(nv.library_path())
    nv.load_library()


def test_every_declared_symbol_is_exported():
    lib = nv.load_library()
    syms = declared_symbols()
    assert len(syms) >= 12
    for s in syms:
        assert hasattr(lib, s), f"{s} declared in nvfp4.h but not exported"


def test_binding_covers_every_symbol():
    assert set(declared_symbols()) == set(nv._SIGNATURES)


def test_version_and_status_strings():
    lib = nv.load_library()
    assert nv.abi_version() == nv.ABI_VERSION
    with open(HEADER) as f:
        assert f"#define NVFP4_ABI_VERSION {nv.ABI_VERSION}\n" in f.read()
    for code in range(8):
        assert lib.nvfp4_status_string(code)
    assert b"unknown" in lib.nvfp4_status_string(99)


def _w(n=64, k=128, groups=1, codes=A, scales=A, s2=A, layout=0):
    return nv._Weight(codes, scales, s2, n, k, groups, layout)


def P(v):
    return ctypes.c_void_p(v)


@pytest.mark.parametrize("kw,status", [
    (dict(k=48), ESHAPE), (dict(k=16), ESHAPE), (dict(k=0), ESHAPE), (dict(n=0), ESHAPE),
    (dict(groups=0), ESHAPE), (dict(codes=0), ENULL), (dict(scales=0), ENULL), (dict(s2=0), ENULL),
    (dict(codes=A + 4), EALIGN), (dict(scales=A + 8), EALIGN), (dict(groups=2), ESHAPE),
    (dict(layout=2), ESHAPE), (dict(layout=1), ESHAPE),            # tiled needs k % 256 == 0
    (dict(layout=1, n=48, k=256), ESHAPE),                        # ... and n % 32 == 0
])
def test_linear_rejects_bad_weight(kw, status):
    lib = nv.load_library()
    w = _w(**kw)
    assert lib.nvfp4_linear(P(A), 4, ctypes.byref(w), P(B), None) == status


def test_linear_rejects_bad_activations():
    lib = nv.load_library()
    w = _w()
    assert lib.nvfp4_linear(P(0), 4, ctypes.byref(w), P(B), None) == ENULL
    assert lib.nvfp4_linear(P(A), 4, ctypes.byref(w), P(0), None) == ENULL
    assert lib.nvfp4_linear(P(A + 2), 4, ctypes.byref(w), P(B), None) == EALIGN
    assert lib.nvfp4_linear(P(A), -1, ctypes.byref(w), P(B), None) == ESHAPE
    assert lib.nvfp4_linear(P(A), 4, None, P(B), None) == ENULL
    # m == 0 is a successful no-op (nothing enqueued)
    assert lib.nvfp4_linear(P(0), 0, ctypes.byref(w), P(0), None) == OK


def test_linear_gated_rejects_mismatched_up():
    lib = nv.load_library()
    g, u = _w(n=64), _w(n=32)
    assert lib.nvfp4_linear_gated(P(A), 4, ctypes.byref(g), ctypes.byref(u), P(B), None) == ESHAPE
    assert lib.nvfp4_linear_gated(P(A), 4, ctypes.byref(g), None, P(B), None) == ENULL


def test_pack_validation():
    lib = nv.load_library()
    ws = lib.nvfp4_pack_workspace_size(3, 64, 128)
    assert ws > 0
    args = lambda **o: [P(o.get("w", A)), o.get("batch", 3), o.get("n", 64), o.get("k", 128), P(o.get("codes", A)),
                        P(o.get("scales", A)), P(o.get("s2", A)), P(o.get("ws", B)), o.get("wsb", ws),
                        o.get("layout", 0), None]
    assert lib.nvfp4_pack(*args(k=40)) == ESHAPE
    assert lib.nvfp4_pack(*args(batch=0)) == ESHAPE
    assert lib.nvfp4_pack(*args(w=0)) == ENULL
    assert lib.nvfp4_pack(*args(codes=A + 1)) == EALIGN
    assert lib.nvfp4_pack(*args(wsb=ws - 1)) == EWS
    assert lib.nvfp4_pack(*args(ws=0)) == EWS
    assert lib.nvfp4_pack(*args(layout=1)) == ESHAPE          # tiled: k % 256 != 0
    assert lib.nvfp4_pack(*args(layout=1, k=256, n=40, wsb=lib.nvfp4_pack_workspace_size(3, 40, 256))) == ESHAPE
    assert lib.nvfp4_pack(*args(layout=7)) == ESHAPE


def test_relayout_validation():
    lib = nv.load_library()
    src, dst = _w(n=64, k=256), _w(n=64, k=256, layout=1, codes=B, scales=B)
    assert lib.nvfp4_relayout(ctypes.byref(src), None, None) == ENULL
    bad = _w(n=32, k=256, layout=1, codes=B, scales=B)
    assert lib.nvfp4_relayout(ctypes.byref(src), ctypes.byref(bad), None) == ESHAPE
    odd = _w(n=64, k=128, layout=1, codes=B, scales=B)
    assert lib.nvfp4_relayout(ctypes.byref(_w(n=64, k=128)), ctypes.byref(odd), None) == ESHAPE
    # same layout and same buffers: nothing to do
    assert lib.nvfp4_relayout(ctypes.byref(src), ctypes.byref(src), None) == OK


def test_dequant_validation():
    lib = nv.load_library()
    w = _w()
    assert lib.nvfp4_dequant(ctypes.byref(w), P(0), P(0), None) == ENULL
    assert lib.nvfp4_dequant(ctypes.byref(w), P(A + 2), P(0), None) == EALIGN
    bad = _w(k=40)
    assert lib.nvfp4_dequant(ctypes.byref(bad), P(A), P(0), None) == ESHAPE


def test_route_validation():
    lib = nv.load_library()
    assert lib.nvfp4_moe_route(P(A), 4, 0, 16, 0, P(A), P(A), P(A), P(0), 0, None) == ESHAPE
    assert lib.nvfp4_moe_route(P(A), 4, 65, 16, 0, P(A), P(A), P(A), P(0), 0, None) == ESHAPE
    assert lib.nvfp4_moe_route(P(A), 4, 8, 0, 0, P(A), P(A), P(A), P(0), 0, None) == ESHAPE
    assert lib.nvfp4_moe_route(P(A), 4, 8, 4097, 0, P(A), P(A), P(A), P(0), 0, None) == ESHAPE
    assert lib.nvfp4_moe_route(P(A), 4, 8, 16, 0, P(0), P(A), P(A), P(0), 0, None) == ENULL
    assert lib.nvfp4_moe_route(P(0), 4, 8, 16, 0, P(A), P(A), P(A), P(0), 0, None) == ENULL


def _moe(lib, T=8, H=256, k=4, E=16, I=128, eb=0, x=A, ids=A, tw=A, y=B, ws=B, wsb=None, **wo):
    g = _w(n=wo.get("gn", I), k=wo.get("gk", H), groups=wo.get("gg", E), layout=wo.get("gl", 0))
    u = _w(n=wo.get("un", I), k=wo.get("uk", H), groups=wo.get("ug", E), layout=wo.get("ul", 0))
    d = _w(n=wo.get("dn", H), k=wo.get("dk", I), groups=wo.get("dg", E), layout=wo.get("dl", 0))
    if wsb is None:
        wsb = lib.nvfp4_moe_workspace_size(T, k, E, H, I)
    return lib.nvfp4_moe_grouped(P(x), T, H, P(ids), P(tw), k, eb, ctypes.byref(g), ctypes.byref(u),
                                 ctypes.byref(d), P(ws), wsb, P(y), None)


def test_moe_validation():
    lib = nv.load_library()
    assert _moe(lib, gk=128) == ESHAPE            # gate k != H
    assert _moe(lib, un=64) == ESHAPE             # up n != I
    assert _moe(lib, dn=128) == ESHAPE            # down n != H
    assert _moe(lib, dk=64) == ESHAPE             # down k != I
    assert _moe(lib, ug=8) == ESHAPE              # expert counts differ
    assert _moe(lib, k=0) == ESHAPE
    assert _moe(lib, k=65) == ESHAPE
    assert _moe(lib, T=-1) == ESHAPE
    assert _moe(lib, H=48, gk=48, uk=48, dn=48) == ESHAPE   # H % 32 != 0
    assert _moe(lib, x=0) == ENULL
    assert _moe(lib, ids=0) == ENULL
    assert _moe(lib, tw=0) == ENULL
    assert _moe(lib, x=A + 2) == EALIGN
    assert _moe(lib, ws=0) == EWS
    assert _moe(lib, wsb=lib.nvfp4_moe_workspace_size(8, 4, 16, 256, 128) - 1) == EWS
    assert _moe(lib, E=4097) == ESHAPE
    assert _moe(lib, gl=1, ul=0, H=256, I=256, gn=256, un=256, dk=256) == ESHAPE   # gate and up layouts differ
    assert _moe(lib, dl=1) == ESHAPE              # tiled down needs k = I % 256 == 0


def _moe_w4a4(lib, s_gu=A, s_d=A + 4, T=8, H=256, k=4, E=16, I=128, **kw):
    g = _w(n=I, k=H, groups=E)
    u = _w(n=I, k=H, groups=E)
    d = _w(n=H, k=I, groups=E)
    wsb = kw.get("wsb", lib.nvfp4_moe_workspace_size(T, k, E, H, I))
    return lib.nvfp4_moe_grouped_w4a4(P(kw.get("x", A)), T, H, P(A), P(A), k, 0, ctypes.byref(g), ctypes.byref(u),
                                      ctypes.byref(d), P(s_gu), P(s_d), P(kw.get("ws", B)), wsb, P(B), None)


def test_moe_w4a4_validation():
    lib = nv.load_library()
    assert _moe_w4a4(lib, s_gu=0) == ENULL
    assert _moe_w4a4(lib, s_d=0) == ENULL
    assert _moe_w4a4(lib, x=0) == ENULL
    assert _moe_w4a4(lib, ws=0) == EWS
    assert _moe_w4a4(lib, T=0, wsb=0) == OK


def test_quantize_act_validation():
    lib = nv.load_library()
    q = lambda x=A, rows=4, k=64, s=A, c=B, sc=B + 4096: lib.nvfp4_quantize_act(P(x), rows, k, P(s), P(c), P(sc), None)
    assert q(k=48) == ESHAPE
    assert q(k=16) == ESHAPE
    assert q(rows=-1) == ESHAPE
    assert q(rows=0, x=0) == OK
    assert q(x=0) == ENULL
    assert q(s=0) == ENULL
    assert q(c=0) == ENULL
    assert q(x=A + 2) == EALIGN
    assert q(sc=B + 4098) == EALIGN
    assert q(s=A + 2) == EALIGN


def test_moe_empty_batch_is_noop():
    lib = nv.load_library()
    assert _moe(lib, T=0, x=0, ids=0, tw=0, y=0, ws=0, wsb=0) == OK


def test_workspace_sizes_monotone_and_cover_buffers():
    lib = nv.load_library()
    a = lib.nvfp4_moe_workspace_size(64, 8, 288, 4096, 1536)
    b = lib.nvfp4_moe_workspace_size(4096, 8, 288, 4096, 1536)
    S = 4096 * 8
    assert b > a > 0
    assert b >= S * 1536 * 2 + S * 4096 * 4          # H (bf16) and Ypart (fp32)
    assert lib.nvfp4_moe_workspace_size(0, 8, 288, 4096, 1536) > 0
    assert lib.nvfp4_moe_workspace_size(4, 0, 288, 4096, 1536) == 0


def test_selftest_fp4_convert_validation():
    # argument errors return before any launch (no device needed)
    lib = nv.load_library()
    assert lib.nvfp4_selftest_fp4_convert(None, None) == ENULL
    assert lib.nvfp4_selftest_fp4_convert(P(A + 4), None) == EALIGN


def test_route_workspace_size():
    # no scratch up to 4096 slots (one workgroup routes them); beyond, one row of
    # per-expert counts per window of >= 2048 slots, at most 64 windows; the routed
    # MLP keeps them in its fp32 partials, which are always large enough
    lib = nv.load_library()
    f = lib.nvfp4_moe_route_workspace_size
    assert f(512, 8, 288) == 0
    assert f(4096 // 8, 8, 288) == 0
    assert f(4096 // 8 + 1, 8, 288) == 3 * 288 * 4          # 4104 slots: 3 windows of 2048
    assert f(4096, 8, 288) == 16 * 288 * 4                  # 32768 slots: 16 windows
    assert f(16500, 8, 288) == 63 * 288 * 4                 # 132000 slots: 63 windows of 2112
    assert f(1 << 20, 8, 4096) == 64 * 4096 * 4
    assert f(-1, 8, 288) == 0 and f(4, 0, 288) == 0 and f(4, 8, 0) == 0
    for T in (513, 4096, 16500, 1 << 20):
        for E in (1, 288, 4096):
            if f(T, 8, E):
                assert f(T, 8, E) <= T * 8 * 32 * 4           # the smallest Ypart (H = 32) holds them


def test_block_validation():
    lib = nv.load_library()
    r = lambda T=4, H=256, E=16, k=2, ws=B, wsb=None, x=A, ids=B, w=B + 4096: lib.nvfp4_router_topk(
        P(x), T, H, P(A), E, k, P(ws), lib.nvfp4_router_workspace_size(T, H, E) if wsb is None else wsb, P(ids), P(w),
        None)
    assert r(H=48) == ESHAPE                 # H % 32
    assert r(E=18) == ESHAPE                 # E % 4
    assert r(k=17) == ESHAPE                 # k > E
    assert r(k=0) == ESHAPE
    assert r(T=0, x=0) == OK
    assert r(x=0) == ENULL
    assert r(x=A + 2) == EALIGN
    assert r(ids=B + 2) == EALIGN
    assert r(wsb=16) == EWS
    m = lambda M=4, H=256, Is=128, ws=B, wsb=None, y=B: lib.nvfp4_bf16_mlp(
        P(A), M, H, P(A), P(A), P(A), Is, P(ws), lib.nvfp4_bf16_mlp_workspace_size(M, H, Is) if wsb is None else wsb,
        P(y), None)
    assert m(Is=100) == ESHAPE
    assert m(H=40) == ESHAPE
    assert m(M=0) == OK
    assert m(y=0) == ENULL
    assert m(y=B + 8) == EALIGN
    assert m(wsb=8) == EWS
    gw = _w(n=128, k=256, groups=16)
    dw = _w(n=256, k=128, groups=16)
    blk = lambda T=8, k=4, Is=128, wsb=None, sg=A: lib.nvfp4_moe_block(
        P(A), T, 256, P(A), k, ctypes.byref(gw), ctypes.byref(gw), ctypes.byref(dw), P(sg), P(A), P(A), Is, P(B),
        lib.nvfp4_moe_block_workspace_size(T, k, 16, 256, 128, Is) if wsb is None else wsb, P(B), None)
    assert blk(k=17) == ESHAPE
    assert blk(Is=100) == ESHAPE
    assert blk(sg=0) == ENULL
    assert blk(wsb=64) == EWS
    assert blk(T=0) == OK


@pytest.mark.parametrize("gate,up,down", [
    (dict(n=128, k=256), dict(n=64, k=256), dict(n=256, k=128)),      # up n != I
    (dict(n=128, k=256), dict(n=128, k=256), dict(n=256, k=64)),      # down k != I
    (dict(n=128, k=256), dict(n=128, k=256), dict(n=128, k=128)),     # down n != H
    (dict(n=256, k=256), dict(n=256, k=256, layout=1), dict(n=256, k=256)),   # gate and up layouts differ
    (dict(n=128, k=256), dict(n=128, k=256, groups=8), dict(n=256, k=128)),   # expert counts differ
])
def test_block_rejects_bad_routed_weights_before_any_launch(gate, up, down):
    # the routed part's checks run before the router is enqueued: with no GPU here, a
    # launch would come back as NVFP4_ERR_HIP instead of the shape error
    lib = nv.load_library()
    g = _w(**{"groups": 16, **gate})
    u = _w(**{"groups": 16, **up})
    d = _w(**{"groups": 16, **down})
    I = gate["n"]
    wsb = lib.nvfp4_moe_block_workspace_size(8, 4, 16, 256, I, 128)
    st = lib.nvfp4_moe_block(P(A), 8, 256, P(A), 4, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), P(A), P(A),
                             P(A), 128, P(B), wsb, P(B), None)
    assert st == ESHAPE


def _moe_class(lib, cls, T=8, H=256, k=4, E=16, I=128, **kw):
    g, u, d = _w(n=I, k=H, groups=E), _w(n=I, k=H, groups=E), _w(n=H, k=I, groups=E)
    wsb = kw.get("wsb", lib.nvfp4_moe_workspace_size(T, k, E, H, I))
    return lib.nvfp4_moe_grouped_class(P(kw.get("x", A)), T, H, P(A), P(A), k, 0, ctypes.byref(g), ctypes.byref(u),
                                       ctypes.byref(d), cls, P(kw.get("ws", B)), wsb, P(B), None)


def test_moe_class_validation():
    lib = nv.load_library()
    assert _moe_class(lib, 3) == EUNSUP
    assert _moe_class(lib, -1) == EUNSUP
    for cls in (0, 1, 2):
        assert _moe_class(lib, cls, x=0) == ENULL
        assert _moe_class(lib, cls, ws=0) == EWS
        assert _moe_class(lib, cls, T=0, wsb=0) == OK


def _plan(lib, T, k, E, H, I, gl=1, dl=1, cls=0):
    out = (ctypes.c_int32 * 5)()
    st = lib.nvfp4_moe_plan(T, k, E, H, I, gl, dl, cls, out)
    return st, tuple(out)


DEC_K, DEC, RES, PRE, FB, TINY = 1, 2, 3, 4, 5, 6


def test_moe_plan_names_the_kernels():
    # without a GPU the library takes 256 compute units, the MI355X's count
    lib = nv.load_library()
    layer = (8, 288, 4096, 1536)
    assert _plan(lib, 1, *layer) == (OK, (4, TINY, TINY, 0, 1))
    assert _plan(lib, 3, *layer) == (OK, (4, TINY, TINY, 0, 1))
    assert _plan(lib, 4, *layer) == (OK, (4, DEC_K, RES, 2, 1))
    # 5 tokens (40 slots) leave the 4-row tiles; 4 tokens of top-16 (64 slots) too
    assert _plan(lib, 5, *layer) == (OK, (16, DEC, RES, 2, 1))
    assert _plan(lib, 4, 16, 288, 4096, 1536) == (OK, (16, DEC, RES, 4, 1))
    # 3 tokens of top-8 with I = 192 (a tensor-parallel shard): K-split gate/up, decode down
    assert _plan(lib, 3, 8, 288, 4096, 192, 0, 0) == (OK, (4, DEC_K, DEC, 0, 1))
    assert _plan(lib, 16, *layer) == (OK, (16, DEC, RES, 4, 1))
    assert _plan(lib, 64, *layer) == (OK, (16, DEC, RES, 4, 1))
    assert _plan(lib, 4096, *layer) == (OK, (128, PRE, PRE, 2, 1))
    # a pinned class overrides the batch-size rule
    assert _plan(lib, 1, *layer, cls=2) == (OK, (128, PRE, PRE, 1, 1))
    assert _plan(lib, 4096, *layer, cls=1) == (OK, (16, DEC, RES, 4, 1))
    assert _plan(lib, 1, *layer, cls=1) == (OK, (16, DEC, RES, 1, 1))
    # row-major weights of shapes the fast kernels do not cover: the fallback, bf16 operands
    assert _plan(lib, 9, 2, 3, 96, 64, 0, 0) == (OK, (16, FB, FB, 0, 0))
    # tiled weights must have shapes the tiled layout allows
    assert _plan(lib, 9, 2, 3, 96, 64)[0] == ESHAPE
    assert _plan(lib, 9, 2, 3, 96, 64, 0, 0, cls=7)[0] == EUNSUP
    assert lib.nvfp4_moe_plan(8, 2, 3, 256, 256, 0, 0, 0, None) == ENULL


def test_moe_grouped_bf16_validation():
    lib = nv.load_library()
    f = lambda T=8, H=256, k=2, E=4, I=128, x=A, wsb=None, ws=B: lib.nvfp4_moe_grouped_bf16(
        P(x), T, H, P(A), P(A), k, 0, P(A), P(A), P(A), E, I, P(ws),
        lib.nvfp4_moe_grouped_bf16_workspace_size(T, k, E, H, I) if wsb is None else wsb, P(B), None)
    assert f(I=100) == ESHAPE
    assert f(H=96) == ESHAPE
    assert f(k=0) == ESHAPE
    assert f(E=0) == ESHAPE
    assert f(T=0, x=0) == OK
    assert f(x=0) == ENULL
    assert f(x=A + 2) == EALIGN
    assert f(wsb=64) == EWS


def _noalloc(lib, T=8, H=256, k=4, E=16, I=128, x=A, y=B, **wo):
    g = _w(n=wo.get("gn", I), k=H, groups=E)
    u = _w(n=I, k=H, groups=E)
    d = _w(n=H, k=I, groups=E)
    return lib.nvfp4_moe_grouped_noalloc(P(x), T, H, P(A), P(A), k, 0, ctypes.byref(g), ctypes.byref(u),
                                         ctypes.byref(d), P(y), None)


def test_moe_noalloc_validation_and_scratch_limit():
    # every check runs on the host before the scratch is looked up or anything is enqueued
    lib = nv.load_library()
    assert _noalloc(lib, gn=64) == ESHAPE
    assert _noalloc(lib, x=0) == ENULL
    assert _noalloc(lib, y=B + 2) == EALIGN
    assert _noalloc(lib, T=0, x=0, y=0) == OK
    # the fixed scratch holds a 256-token top-8 step of the 288-expert layer, not a 4096-token one
    layer = dict(H=4096, I=1536, E=288, k=8)
    assert lib.nvfp4_moe_workspace_size(256, 8, 288, 4096, 1536) <= nv.NOALLOC_SCRATCH_BYTES
    assert lib.nvfp4_moe_workspace_size(4096, 8, 288, 4096, 1536) > nv.NOALLOC_SCRATCH_BYTES
    assert _noalloc(lib, T=4096, **layer) == ESCRATCH
