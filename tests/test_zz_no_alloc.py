"""The no-allocation entry point (nvfp4_moe_grouped_noalloc) against the
entry point with a caller workspace (nvfp4_moe_grouped), through the C ABI.

Both run the same kernels, so their outputs must be equal bit for bit; each
must also meet the oracle's bar. Two calls in a row share the library's fixed
scratch, the second on a smaller batch (and a different kernel class) than the
first; a third call repeats the first over the second's leftovers, and a fourth
takes two tokens through the two-launch path for tiny batches."""
import ctypes

import numpy as np
import pytest
import torch

import nvfp4_moe_expert_amd as nv
import synth
from gpu_util import DEV, assert_close, bf16_dev, bf16_host_bits, bf16_host_f64, note, weight_dev
from oracle import mlp as OM
from oracle import nvfp4 as ONV

pytestmark = pytest.mark.gpu

K_TOP, E, H, I = 8, 32, 1024, 512


@pytest.fixture(scope="module")
def weights():
    packs = [ONV.pack_batch(synth.expert_weights(E, n, kk, 0.05, 150, st))
             for n, kk, st in ((I, H, synth.S_GATE), (I, H, synth.S_UP), (H, I, synth.S_DOWN))]
    return packs, [weight_dev(p, nv.LAYOUT_TILED32) for p in packs]


def _inputs(T, seed):
    x = synth.bf16_normal((T, H), 1.0, seed, synth.S_X)
    ids, w = synth.topk_softmax_routing(T, E, K_TOP, seed, synth.S_ROUTE)
    return x, ids.astype(np.int32), w.astype(np.float32)


def _noalloc_c(xd, idd, wd, dev_w, y):
    """nvfp4_moe_grouped_noalloc called through ctypes on the C ABI directly."""
    lib = nv.load_library()
    T, Hh = xd.shape
    g, u, d = (w._struct() for w in dev_w)
    st = lib.nvfp4_moe_grouped_noalloc(ctypes.c_void_p(xd.data_ptr()), T, Hh, ctypes.c_void_p(idd.data_ptr()),
                                       ctypes.c_void_p(wd.data_ptr()), K_TOP, 0, ctypes.byref(g), ctypes.byref(u),
                                       ctypes.byref(d), ctypes.c_void_p(y.data_ptr()),
                                       ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, f"nvfp4_moe_grouped_noalloc: status {st}"


def test_noalloc_equals_workspace_entry_point_on_consecutive_calls(weights):
    packs, dev_w = weights
    results = []
    for T, seed in ((96, 151), (5, 152), (96, 151), (2, 154)):
        plan = nv.moe_plan(T, K_TOP, E, H, I, nv.LAYOUT_TILED32, nv.LAYOUT_TILED32)
        note(f"noalloc T={T}: {plan}")
        x, ids, w = _inputs(T, seed)
        xd, idd, wd = bf16_dev(x), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV)
        y = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device=DEV)
        _noalloc_c(xd, idd, wd, dev_w, y)
        ref = nv.moe_grouped(xd, idd, wd, *dev_w)
        torch.cuda.synchronize()
        assert np.array_equal(bf16_host_bits(y), bf16_host_bits(ref)), f"T={T}: differs from nvfp4_moe_grouped"
        assert_close(bf16_host_f64(y), OM.moe(x, ids, w, *packs), f"noalloc T={T}")
        results.append(bf16_host_bits(y))
    assert np.array_equal(results[0], results[2])


def test_noalloc_binding_and_scratch_limit(weights):
    _, dev_w = weights
    x, ids, w = _inputs(3, 153)
    out = torch.empty((3, H), dtype=torch.bfloat16, device=DEV)
    y = nv.moe_grouped_noalloc(bf16_dev(x), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV), *dev_w, out=out)
    ref = nv.moe_grouped(bf16_dev(x), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV), *dev_w)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_host_bits(y), bf16_host_bits(ref))
    # a batch whose workspace exceeds the fixed scratch is refused on the host
    T = 4096
    assert nv.moe_workspace_size(T, K_TOP, E, H, I) > nv.NOALLOC_SCRATCH_BYTES
    xb = torch.zeros((T, H), dtype=torch.bfloat16, device=DEV)
    ib = torch.zeros((T, K_TOP), dtype=torch.int32, device=DEV)
    wb = torch.zeros((T, K_TOP), dtype=torch.float32, device=DEV)
    with pytest.raises(nv.Nvfp4Error) as exc:
        nv.moe_grouped_noalloc(xb, ib, wb, *dev_w, out=torch.empty((T, H), dtype=torch.bfloat16, device=DEV))
    assert exc.value.status == 7
