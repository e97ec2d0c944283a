"""Out-of-bounds guards and the fp16 form's dynamic range, on the GPU.

Guards: every entry point writes its outputs (and, where it takes one, uses
its workspace) inside buffers that are fenced on both sides by sentinel bytes;
after the call the fences must be untouched. Shapes have ragged tails (rows,
columns and slots that are not multiples of the kernels' tiles), and the
routed MLP is run in each kernel class.

Dynamic range: the routed kernels feed fp16 operands after scaling each
activation row by a power of two (include/nvfp4.h, Numerics). Rows whose
magnitudes span 2^-24 .. 2^24, with a wide spread inside each row, must still
meet the oracle's bar row by row (a global bar would hide a small row that went
wrong)."""
import ctypes

import numpy as np
import pytest
import torch

import nvfp4_moe_expert_amd as nv
import synth
from gpu_util import DEV, assert_close, bf16_dev, bf16_host_f64, note, weight_dev
from oracle import mlp as OM
from oracle import nvfp4 as ONV

pytestmark = pytest.mark.gpu

FENCE = 512          # bytes of sentinel on each side
SENT = 0xA5


class Fenced:
    """A device buffer of `nbytes` with FENCE sentinel bytes before and after."""

    def __init__(self, nbytes, dtype=torch.uint8, shape=None, fill=SENT):
        self.nbytes = int(nbytes)
        self.raw = torch.full((self.nbytes + 2 * FENCE,), SENT, dtype=torch.uint8, device=DEV)
        inner = self.raw[FENCE:FENCE + self.nbytes]
        if fill != SENT:
            inner.fill_(fill)
        self.t = inner.view(dtype)
        if shape is not None:
            self.t = self.t.view(shape)

    @property
    def ptr(self):
        return ctypes.c_void_p(self.t.data_ptr())

    def check(self, what):
        b = self.raw.cpu().numpy()
        assert np.all(b[:FENCE] == SENT), f"{what}: bytes written before the buffer"
        assert np.all(b[FENCE + self.nbytes:] == SENT), f"{what}: bytes written past the buffer"


def _s():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ok(st, where):
    assert st == 0, f"{where}: status {st}"


def _wstruct(codes, scales, s2, n, k, g, layout):
    return nv._Weight(codes.data_ptr(), scales.data_ptr(), s2.data_ptr(), n, k, g, layout)


@pytest.mark.parametrize("layout", [nv.LAYOUT_ROWS, nv.LAYOUT_TILED32])
def test_pack_relayout_dequant_stay_inside(layout):
    lib = nv.load_library()
    G, N, K = 3, 96, 512
    w = bf16_dev(np.stack([synth.bf16_normal((N, K), 0.02, 140, g) for g in range(G)]))
    codes, scales, s2 = Fenced(G * N * K // 2), Fenced(G * N * K // 16), Fenced(4 * G, torch.float32)
    wsb = lib.nvfp4_pack_workspace_size(G, N, K)
    ws = Fenced(wsb)
    _ok(lib.nvfp4_pack(ctypes.c_void_p(w.data_ptr()), G, N, K, codes.ptr, scales.ptr, s2.ptr, ws.ptr, wsb, layout,
                       _s()), "pack")
    other = nv.LAYOUT_ROWS if layout == nv.LAYOUT_TILED32 else nv.LAYOUT_TILED32
    rc, rs = Fenced(G * N * K // 2), Fenced(G * N * K // 16)
    src = _wstruct(codes.t, scales.t, s2.t, N, K, G, layout)
    dst = _wstruct(rc.t, rs.t, s2.t, N, K, G, other)
    _ok(lib.nvfp4_relayout(ctypes.byref(src), ctypes.byref(dst), _s()), "relayout")
    u, f = Fenced(2 * G * N * K), Fenced(4 * G * N * K)
    _ok(lib.nvfp4_dequant(ctypes.byref(src), u.ptr, f.ptr, _s()), "dequant")
    torch.cuda.synchronize()
    for b, n in ((codes, "codes"), (scales, "scales"), (s2, "scale_2"), (ws, "pack workspace"), (rc, "relayout codes"),
                 (rs, "relayout scales"), (u, "dequant bf16"), (f, "dequant fp32")):
        b.check(n)


@pytest.mark.parametrize("M,N,K,layout", [(5, 128, 512, 0), (37, 96, 512, 1), (37, 96, 256, 0), (300, 160, 512, 1),
                                           (3, 48, 96, 0)])
def test_linear_and_gated_stay_inside(M, N, K, layout):
    lib = nv.load_library()
    x = bf16_dev(synth.bf16_normal((M, K), 1.0, 141, M))
    wg = weight_dev(ONV.pack(synth.bf16_normal((N, K), 0.05, 141, 1)), layout)
    wu = weight_dev(ONV.pack(synth.bf16_normal((N, K), 0.05, 141, 2)), layout)
    y, h = Fenced(2 * M * N), Fenced(2 * M * N)
    g, u = wg._struct(), wu._struct()
    _ok(lib.nvfp4_linear(ctypes.c_void_p(x.data_ptr()), M, ctypes.byref(g), y.ptr, _s()), "linear")
    _ok(lib.nvfp4_linear_gated(ctypes.c_void_p(x.data_ptr()), M, ctypes.byref(g), ctypes.byref(u), h.ptr, _s()),
        "linear_gated")
    torch.cuda.synchronize()
    y.check("linear y")
    h.check("linear_gated h")


def _moe_inputs(T, k, E, H, I, seed):
    x = synth.bf16_normal((T, H), 1.0, seed, synth.S_X)
    ids, w = synth.topk_softmax_routing(T, E, k, seed, synth.S_ROUTE)
    packs = [ONV.pack_batch(synth.expert_weights(E, n, kk, 0.05, seed, st))
             for n, kk, st in ((I, H, synth.S_GATE), (I, H, synth.S_UP), (H, I, synth.S_DOWN))]
    return x, ids.astype(np.int32), w.astype(np.float32), packs


@pytest.mark.parametrize("T,k,E,H,I,cls,layout", [
    (7, 3, 16, 512, 512, nv.CLASS_AUTO, 1),       # 21 slots: K-split gate/up, resident down
    (37, 3, 8, 512, 512, nv.CLASS_DECODE, 1),     # decode tiles with ragged ends
    (37, 3, 8, 512, 512, nv.CLASS_PREFILL, 1),    # prefill tiles with ragged ends
    (37, 3, 8, 320, 320, nv.CLASS_PREFILL, 0),    # prefill tiles, partial last column block, K ending mid-stage
    (130, 4, 6, 256, 256, nv.CLASS_AUTO, 0),      # prefill, row-major
    (9, 2, 3, 96, 64, nv.CLASS_AUTO, 0),          # the fallback GEMM
])
def test_moe_grouped_output_and_workspace_stay_inside(T, k, E, H, I, cls, layout):
    lib = nv.load_library()
    note(f"guards: moe T={T} k={k} E={E} H={H} I={I} class={cls} layout={layout}")
    x, ids, w, packs = _moe_inputs(T, k, E, H, I, 142 + T)
    xd, idd, wd = bf16_dev(x), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV)
    dev_w = [weight_dev(p, layout) for p in packs]      # kept alive: the structs hold raw pointers
    g, u, d = (dw._struct() for dw in dev_w)
    wsb = lib.nvfp4_moe_workspace_size(T, k, E, H, I)
    ws = Fenced(wsb)
    y = Fenced(2 * T * H, fill=0)
    args = (ctypes.c_void_p(xd.data_ptr()), T, H, ctypes.c_void_p(idd.data_ptr()), ctypes.c_void_p(wd.data_ptr()), k,
            0, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d))
    _ok(lib.nvfp4_moe_grouped_class(*args, cls, ws.ptr, wsb, y.ptr, _s()), "moe_grouped_class")
    torch.cuda.synchronize()
    y.check("moe y")
    ws.check("moe workspace")
    assert_close(bf16_host_f64(y.t.view(torch.bfloat16).view(T, H)), OM.moe(x, ids, w, *packs), "moe guarded")
    # W4A4 on the shapes its kernels cover
    if cls == nv.CLASS_AUTO and H % 256 == 0 and I % 256 == 0:
        sc = torch.tensor([2.0 / 2688, 4.0 / 2688], dtype=torch.float32, device=DEV)
        y4 = Fenced(2 * T * H)
        _ok(lib.nvfp4_moe_grouped_w4a4(*args, ctypes.c_void_p(sc.data_ptr()), ctypes.c_void_p(sc.data_ptr() + 4),
                                       ws.ptr, wsb, y4.ptr, _s()), "moe_grouped_w4a4")
        torch.cuda.synchronize()
        y4.check("w4a4 y")
        ws.check("w4a4 workspace")


def test_route_quantize_router_stay_inside():
    lib = nv.load_library()
    T, k, E, H = 37, 3, 20, 256
    ids = np.random.default_rng(143).integers(-2, E + 3, (T, k)).astype(np.int32)
    idd = torch.from_numpy(ids).to(DEV)
    off, perm, inv = Fenced(4 * (E + 1)), Fenced(4 * T * k), Fenced(4 * T * k)
    _ok(lib.nvfp4_moe_route(ctypes.c_void_p(idd.data_ptr()), T, k, E, 0, off.ptr, perm.ptr, inv.ptr, None, 0, _s()),
        "route")
    x = bf16_dev(synth.bf16_normal((T, H), 1.0, 143))
    sc = torch.tensor([3.0 / 2688], dtype=torch.float32, device=DEV)
    qc, qs = Fenced(T * H // 2), Fenced(T * H // 16)
    _ok(lib.nvfp4_quantize_act(ctypes.c_void_p(x.data_ptr()), T, H, ctypes.c_void_p(sc.data_ptr()), qc.ptr, qs.ptr,
                               _s()), "quantize_act")
    wr = bf16_dev(synth.bf16_normal((E, H), 0.02, 143, 1))
    rwsb = lib.nvfp4_router_workspace_size(T, H, E)
    rws, rid, rw = Fenced(rwsb), Fenced(4 * T * k), Fenced(4 * T * k)
    _ok(lib.nvfp4_router_topk(ctypes.c_void_p(x.data_ptr()), T, H, ctypes.c_void_p(wr.data_ptr()), E, k, rws.ptr, rwsb,
                              rid.ptr, rw.ptr, _s()), "router_topk")
    torch.cuda.synchronize()
    for b, n in ((off, "offsets"), (perm, "perm"), (inv, "inv"), (qc, "act codes"), (qs, "act scales"),
                 (rws, "router workspace"), (rid, "router ids"), (rw, "router weights")):
        b.check(n)


@pytest.mark.parametrize("T", [3, 130])
def test_bf16_mlp_block_and_bf16_experts_stay_inside(T):
    lib = nv.load_library()
    k, E, H, I, Is = 4, 16, 256, 128, 192
    x = bf16_dev(synth.bf16_normal((T, H), 1.0, 144, T))
    xp = ctypes.c_void_p(x.data_ptr())
    sg, su, sd = (bf16_dev(synth.bf16_normal(s, 0.05, 144, 10 + i)) for i, s in enumerate([(Is, H), (Is, H), (H, Is)]))
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    mwsb = lib.nvfp4_bf16_mlp_workspace_size(T, H, Is)
    mws, my = Fenced(mwsb), Fenced(4 * T * H)
    _ok(lib.nvfp4_bf16_mlp(xp, T, H, P(sg), P(su), P(sd), Is, mws.ptr, mwsb, my.ptr, _s()), "bf16_mlp")
    wr = bf16_dev(synth.bf16_normal((E, H), 0.02, 144, 20))
    packs = [ONV.pack_batch(synth.expert_weights(E, n, kk, 0.05, 144, st))
             for n, kk, st in ((I, H, synth.S_GATE), (I, H, synth.S_UP), (H, I, synth.S_DOWN))]
    dev_w = [weight_dev(p) for p in packs]              # kept alive: the structs hold raw pointers
    g, u, d = (dw._struct() for dw in dev_w)
    bwsb = lib.nvfp4_moe_block_workspace_size(T, k, E, H, I, Is)
    bws, by = Fenced(bwsb), Fenced(2 * T * H)
    _ok(lib.nvfp4_moe_block(xp, T, H, P(wr), k, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), P(sg), P(su), P(sd),
                            Is, bws.ptr, bwsb, by.ptr, _s()), "moe_block")
    ids, w = synth.topk_softmax_routing(T, E, k, 144, synth.S_ROUTE)
    idd, wd = torch.from_numpy(ids.astype(np.int32)).to(DEV), torch.from_numpy(w.astype(np.float32)).to(DEV)
    wg, wu, wdn = (bf16_dev(synth.expert_weights(E, n, kk, 0.05, 145, st))
                   for n, kk, st in ((I, H, synth.S_GATE), (I, H, synth.S_UP), (H, I, synth.S_DOWN)))
    ewsb = lib.nvfp4_moe_grouped_bf16_workspace_size(T, k, E, H, I)
    ews, ey = Fenced(ewsb), Fenced(2 * T * H)
    _ok(lib.nvfp4_moe_grouped_bf16(xp, T, H, P(idd), P(wd), k, 0, P(wg), P(wu), P(wdn), E, I, ews.ptr, ewsb, ey.ptr,
                                   _s()), "moe_grouped_bf16")
    torch.cuda.synchronize()
    for b, n in ((mws, "bf16_mlp workspace"), (my, "bf16_mlp y"), (bws, "block workspace"), (by, "block y"),
                 (ews, "bf16 experts workspace"), (ey, "bf16 experts y")):
        b.check(n)


def _wide_rows(T, H, seed):
    """bf16 rows whose scales run from 2^-24 to 2^24 across rows, each row spread
    over about 2^-16 .. 2^4 of its scale."""
    g = np.random.default_rng(seed)
    row_exp = np.linspace(-24, 24, T).round()
    inner = g.standard_normal((T, H)) * np.exp2(g.uniform(-16, 0, (T, H)))
    v = (inner * np.exp2(row_exp)[:, None]).astype(np.float32)
    return synth.f32_to_bf16_bits(v)


@pytest.mark.parametrize("T,k,E,H,I,cls", [
    (7, 4, 8, 512, 512, nv.CLASS_AUTO),          # K-split gate/up, resident down (fp16 H rows)
    (49, 4, 8, 512, 512, nv.CLASS_DECODE),       # decode tiles
    (49, 4, 8, 512, 512, nv.CLASS_PREFILL),      # prefill tiles (fp16 gate/up, bf16 down)
])
def test_fp16_form_wide_dynamic_range_rowwise(T, k, E, H, I, cls):
    note(f"wide-range rows T={T} class={cls}")
    x = _wide_rows(T, H, 146 + T)
    ids, w = synth.topk_softmax_routing(T, E, k, 146, synth.S_ROUTE, T)
    packs = [ONV.pack_batch(synth.expert_weights(E, n, kk, 0.05, 146, st))
             for n, kk, st in ((I, H, synth.S_GATE), (I, H, synth.S_UP), (H, I, synth.S_DOWN))]
    y = nv.moe_grouped(bf16_dev(x), torch.from_numpy(ids.astype(np.int32)).to(DEV),
                       torch.from_numpy(w.astype(np.float32)).to(DEV), *(weight_dev(p, 1) for p in packs),
                       kernel_class=cls)
    torch.cuda.synchronize()
    got = bf16_host_f64(y)
    ref = OM.moe(x, ids, w, *packs)
    assert np.all(np.abs(ref).max(axis=1) > 0)
    for t in range(T):
        assert_close(got[t], ref[t], f"row {t} (scale 2^{np.log2(np.abs(ref[t]).max()):.0f})")
