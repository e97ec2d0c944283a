"""Parity at the full workload sizes, in the launch configuration the benchmark
times, on sampled outputs the oracle computes one by one.

Weights are drawn in bf16 on the device (torch's generator, seeded), packed on
the device by nvfp4_pack, and used by the GPU path. For every expert a sampled
token touches, the oracle packs the same bf16 weights (copied to the host) on
its own; those packs must match the GPU's byte for byte, and the oracle's
routed MLP for the sampled tokens must match the GPU output within the bar.
Properties that hold at any size (token permutation, repeat determinism) are
checked over the whole batch.

The weights are packed in the tiled layout the benchmark uses; the oracle's
row-major packs are compared after the same byte permutation (gpu_util.tile32,
written from the layout's definition).

Workloads:
  decode-shaped MoE layer: 288 experts, top-8, hidden 4096, intermediate 1536,
      T in {1, 16, 64}, routing logits ~ N(0,1), weights ~ N(0, 0.02);
  prefill-shaped MoE layer: same layer, T = 4096, Zipf(1.1)-skewed routing;
  dense Fp4Linear MLP: 2048 tokens, 4096 -> 12288 -> 4096, gate and up with
      distinct scale_2 (gate ~ N(0, 0.02), up ~ N(0, 0.025), down ~ N(0, 0.02));
  W4A4 form of the decode (T = 64) and prefill layers, with fixed activation
      scales of the size a calibration gives for these distributions (x:
      1.05 * 5.0 / 2688 for N(0, 1) rows; H: 1.05 * 8.0 / 2688)."""
import concurrent.futures as cf

import numpy as np
import pytest
import torch

import nvfp4_moe_expert_amd as nv
import synth
from gpu_util import DEV, assert_close, bf16_dev, bf16_host_bits, bf16_host_f64, note, tile32
from oracle import mlp as OM
from oracle import nvfp4 as ONV

pytestmark = pytest.mark.gpu

E, K_TOP, H, I = 288, 8, 4096, 1536
WSEED = 5


@pytest.fixture(scope="module")
def layer():
    """bf16 weights of the 288-expert layer (device) and their GPU packs."""
    note("drawing and packing the 288-expert layer on the device")
    raw = {
        "gate": synth.torch_bf16_normal((E, I, H), 0.02, WSEED * 10 + 1, DEV),
        "up": synth.torch_bf16_normal((E, I, H), 0.02, WSEED * 10 + 2, DEV),
        "down": synth.torch_bf16_normal((E, H, I), 0.02, WSEED * 10 + 3, DEV),
    }
    packed = {k: nv.pack(v, layout=nv.LAYOUT_TILED32) for k, v in raw.items()}
    torch.cuda.synchronize()
    return raw, packed


def _oracle_experts(raw, packed, experts):
    """Oracle packs of the listed experts (threads: numpy releases the GIL), each
    checked byte for byte against the GPU pack."""
    jobs = [(p, e) for e in experts for p in ("gate", "up", "down")]
    host = {(p, e): bf16_host_bits(raw[p][e]) for p, e in jobs}
    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        res = dict(zip(jobs, ex.map(lambda j: ONV.pack(host[j]), jobs)))
    for (p, e), (c, s, s2) in res.items():
        g = packed[p]
        ct, st = tile32(c, s)
        assert np.array_equal(g.codes[e].cpu().numpy(), ct), f"pack codes differ: {p}[{e}]"
        assert np.array_equal(g.scales[e].cpu().numpy(), st), f"pack scales differ: {p}[{e}]"
        assert g.scale_2[e].cpu().numpy().view(np.uint32) == np.float32(s2).view(np.uint32)
    return res


def _oracle_tokens(x, ids, w, res, experts, scales=None):
    """Oracle routed MLP for a few tokens, with the touched experts compacted
    (W4A4 with scales = (input scale of gate/up, of down))."""
    loc = {e: i for i, e in enumerate(experts)}
    lids = np.vectorize(lambda v: loc.get(int(v), -1))(ids).astype(np.int32)
    stack = lambda p: (np.stack([res[(p, e)][0] for e in experts]), np.stack([res[(p, e)][1] for e in experts]),
                       np.array([res[(p, e)][2] for e in experts], np.float32))
    if scales is not None:
        return OM.moe_w4a4(x, lids, w, stack("gate"), stack("up"), stack("down"), *scales)
    return OM.moe(x, lids, w, stack("gate"), stack("up"), stack("down"))


def _moe(x, ids, w, packed, scales=None):
    sc = None if scales is None else torch.tensor(list(scales), dtype=torch.float32, device=DEV)
    return nv.moe_grouped(bf16_dev(x), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV),
                          packed["gate"], packed["up"], packed["down"], input_scales=sc)


W4A4_SCALES = (np.float32(1.05 * 5.0 / 2688), np.float32(1.05 * 8.0 / 2688))


@pytest.mark.parametrize("T,n_sample", [(1, 1), (16, 1), (64, 2)])
def test_decode_layer_sampled(layer, T, n_sample):
    raw, packed = layer
    note(f"decode layer T={T}")
    x = synth.bf16_normal((T, H), 1.0, 3, synth.S_X, T)
    ids, w = synth.topk_softmax_routing(T, E, K_TOP, 3, synth.S_ROUTE, T)
    y = bf16_host_f64(_moe(x, ids, w, packed))
    toks = np.random.default_rng(T).choice(T, n_sample, replace=False)
    experts = sorted(set(ids[toks].ravel().tolist()))
    res = _oracle_experts(raw, packed, experts)
    assert_close(y[toks], _oracle_tokens(x[toks], ids[toks], w[toks], res, experts), f"decode T={T}")


def test_prefill_layer_sampled_and_permutation(layer):
    raw, packed = layer
    T = 4096
    note("prefill layer T=4096 Zipf")
    x = synth.bf16_normal((T, H), 1.0, 4, synth.S_X)
    ids, w = synth.zipf_routing(T, E, K_TOP, 1.1, 4, synth.S_ROUTE)
    y = bf16_host_bits(_moe(x, ids, w, packed))
    # whole-batch properties: repeat and token permutation are bitwise
    assert np.array_equal(bf16_host_bits(_moe(x, ids, w, packed)), y)
    p = np.random.default_rng(9).permutation(T)
    assert np.array_equal(bf16_host_bits(_moe(x[p], ids[p], w[p], packed)), y[p])
    # sampled tokens against the oracle (include one that routes to the busiest expert)
    busiest = np.bincount(ids.ravel(), minlength=E).argmax()
    t0 = int(np.nonzero(np.any(ids == busiest, axis=1))[0][0])
    toks = np.array([t0, T - 1])
    experts = sorted(set(ids[toks].ravel().tolist()))
    res = _oracle_experts(raw, packed, experts)
    yf = bf16_host_f64(torch.from_numpy(y.view(np.int16)).view(torch.bfloat16))
    assert_close(yf[toks], _oracle_tokens(x[toks], ids[toks], w[toks], res, experts), "prefill")


def test_dense_mlp_sampled_rows():
    note("dense MLP 2048 x 4096 -> 12288 -> 4096")
    M, D, F = 2048, 4096, 12288
    raw = {"gate": synth.torch_bf16_normal((F, D), 0.02, 51, DEV),
           # a different sigma for up: with equal sigmas over 50M draws the bf16 amax, and
           # with it scale_2, usually coincides; the workload wants them distinct
           "up": synth.torch_bf16_normal((F, D), 0.025, 52, DEV),
           "down": synth.torch_bf16_normal((D, F), 0.02, 53, DEV)}
    packed = {k: nv.pack(v, layout=nv.LAYOUT_TILED32) for k, v in raw.items()}
    x = synth.bf16_normal((M, D), 1.0, 5, synth.S_X)
    h = nv.linear_gated(bf16_dev(x), packed["gate"], packed["up"])
    y = nv.linear(h, packed["down"])
    torch.cuda.synchronize()
    with cf.ThreadPoolExecutor(max_workers=3) as ex:
        res = dict(zip(raw, ex.map(lambda k: ONV.pack(bf16_host_bits(raw[k])), raw)))
    assert packed["gate"].scale_2.item() != packed["up"].scale_2.item()
    for k, (c, s, s2) in res.items():
        ct, st = tile32(c, s)
        assert np.array_equal(packed[k].codes[0].cpu().numpy(), ct), k
        assert np.array_equal(packed[k].scales[0].cpu().numpy(), st), k
        assert packed[k].scale_2[0].cpu().numpy().view(np.uint32) == np.float32(s2).view(np.uint32)
    rows = np.array([0, 777, M - 1])
    h_ref = OM.linear_gated(x[rows], res["gate"], res["up"])
    assert_close(bf16_host_f64(h)[rows], h_ref, "dense gated")
    y_ref = OM.dense_mlp(x[rows], res["gate"], res["up"], res["down"])
    assert_close(bf16_host_f64(y)[rows], y_ref, "dense MLP")


def test_pack_of_288_expert_projections_sampled(layer):
    # the load-time pack of the 288 experts x 3 projections; a sample of tensors
    # from each projection is re-packed by the oracle
    raw, packed = layer
    experts = [0, 1, 143, 287]
    _oracle_experts(raw, packed, experts)


@pytest.mark.parametrize("T", [64, 4096])
def test_w4a4_layer_sampled(layer, T):
    raw, packed = layer
    note(f"W4A4 layer T={T}")
    if T == 4096:
        x = synth.bf16_normal((T, H), 1.0, 4, synth.S_X)
        ids, w = synth.zipf_routing(T, E, K_TOP, 1.1, 4, synth.S_ROUTE)
    else:
        x = synth.bf16_normal((T, H), 1.0, 3, synth.S_X, T)
        ids, w = synth.topk_softmax_routing(T, E, K_TOP, 3, synth.S_ROUTE, T)
    y = bf16_host_f64(_moe(x, ids, w, packed, W4A4_SCALES))
    toks = np.array([0, T - 1])
    experts = sorted(set(ids[toks].ravel().tolist()))
    res = _oracle_experts(raw, packed, experts)
    assert_close(y[toks], _oracle_tokens(x[toks], ids[toks], w[toks], res, experts, W4A4_SCALES), f"w4a4 T={T}")
