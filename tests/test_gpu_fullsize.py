"""Parity at the full workload sizes, in the launch configuration the benchmark
times, on every output.

Weights are drawn in bf16 on the device (torch's generator, seeded) and packed
on the device by nvfp4_pack in the tiled layout the benchmark uses. The oracle
packs every one of the 288 experts x 3 projections from host copies of the
same bf16 draws; each pack must equal the GPU's byte for byte (compared after
the layout's byte permutation, gpu_util.tile32, written from its definition),
and the oracle's packs are then the weights of the oracle's routed MLP. Every
token of every batch is compared with the oracle.

The oracle's routed MLP is run on groups of experts in parallel threads: a
token's result is the sum over its k slots, and each group contributes the
slots routed to its experts (the other slots count as skipped), so the groups'
float64 results add up to the whole sum up to float64 rounding.

Workloads:
  decode-shaped MoE layer: 288 experts, top-8, hidden 4096, intermediate 1536,
      T in {1, 16, 64}, routing logits ~ N(0,1), weights ~ N(0, 0.02);
  prefill-shaped MoE layer: same layer, T = 4096, Zipf(1.1)-skewed routing;
      also processed in chunks with the prefill class pinned (bitwise equal);
  dense Fp4Linear MLP: 2048 tokens, 4096 -> 12288 -> 4096, gate and up with
      distinct scale_2 (gate ~ N(0, 0.02), up ~ N(0, 0.025), down ~ N(0, 0.02));
  W4A4 form of the decode (T = 64) and prefill layers, with fixed activation
      scales of the size a calibration gives for these distributions (x:
      1.05 * 5.0 / 2688 for N(0, 1) rows; H: 1.05 * 8.0 / 2688)."""
import concurrent.futures as cf
import os

import numpy as np
import pytest
import torch

import nvfp4_moe_expert_amd as nv
import synth
from gpu_util import DEV, assert_close, bf16_dev, bf16_host_bits, bf16_host_f64, note, tile32
from oracle import mlp as OM
from oracle import nvfp4 as ONV

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

E, K_TOP, H, I = 288, 8, 4096, 1536
WSEED = 5
PROJ = ("gate", "up", "down")
WORKERS = max(1, min(16, len(os.sched_getaffinity(0))))


@pytest.fixture(scope="module")
def layer():
    """bf16 weights of the 288-expert layer (device), their GPU packs (tiled), and
    the oracle's packs of every projection (host, row-major)."""
    note("drawing and packing the 288-expert layer on the device")
    raw = {
        "gate": synth.torch_bf16_normal((E, I, H), 0.02, WSEED * 10 + 1, DEV),
        "up": synth.torch_bf16_normal((E, I, H), 0.02, WSEED * 10 + 2, DEV),
        "down": synth.torch_bf16_normal((E, H, I), 0.02, WSEED * 10 + 3, DEV),
    }
    packed = {k: nv.pack(v, layout=nv.LAYOUT_TILED32) for k, v in raw.items()}
    torch.cuda.synchronize()
    note(f"oracle pack of {3 * E} projections on {WORKERS} threads")
    jobs = [(p, e) for e in range(E) for p in PROJ]

    def one(job):
        p, e = job
        return ONV.pack(bf16_host_bits(raw[p][e]))

    ref = {}
    with cf.ThreadPoolExecutor(max_workers=WORKERS) as ex:
        for i, (job, res) in enumerate(zip(jobs, ex.map(one, jobs))):
            ref[job] = res
            if (i + 1) % 216 == 0:
                note(f"  {i + 1} of {len(jobs)} packed")
    stacked = {p: (np.stack([ref[(p, e)][0] for e in range(E)]), np.stack([ref[(p, e)][1] for e in range(E)]),
                   np.array([ref[(p, e)][2] for e in range(E)], np.float32)) for p in PROJ}
    return raw, packed, stacked


def _oracle_moe(x, ids, w, packs, scales=None):
    """The oracle's routed MLP over all tokens, its experts split into groups run in
    parallel (W4A4 with scales = (input scale of gate/up, of down))."""
    groups = np.array_split(np.arange(E), 2 * WORKERS)

    def part(g):
        e0, e1 = int(g[0]), int(g[-1]) + 1
        sub = {p: tuple(a[e0:e1] for a in packs[p][:2]) + (packs[p][2][e0:e1],) for p in PROJ}
        rows = np.nonzero(np.any((ids >= e0) & (ids < e1), axis=1))[0]
        out = np.zeros((x.shape[0], H))
        if rows.size == 0:
            return out
        if scales is None:
            out[rows] = OM.moe(x[rows], ids[rows], w[rows], sub["gate"], sub["up"], sub["down"], expert_begin=e0)
        else:
            out[rows] = OM.moe_w4a4(x[rows], ids[rows], w[rows], sub["gate"], sub["up"], sub["down"], *scales,
                                    expert_begin=e0)
        return out

    with cf.ThreadPoolExecutor(max_workers=WORKERS) as ex:
        return sum(ex.map(part, groups))


def _moe(x, ids, w, packed, scales=None, kernel_class=None):
    sc = None if scales is None else torch.tensor(list(scales), dtype=torch.float32, device=DEV)
    return nv.moe_grouped(bf16_dev(x), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV),
                          packed["gate"], packed["up"], packed["down"], input_scales=sc, kernel_class=kernel_class)


W4A4_SCALES = (np.float32(1.05 * 5.0 / 2688), np.float32(1.05 * 8.0 / 2688))


def _decode_inputs(T):
    x = synth.bf16_normal((T, H), 1.0, 3, synth.S_X, T)
    ids, w = synth.topk_softmax_routing(T, E, K_TOP, 3, synth.S_ROUTE, T)
    return x, ids, w


def _prefill_inputs():
    T = 4096
    x = synth.bf16_normal((T, H), 1.0, 4, synth.S_X)
    ids, w = synth.zipf_routing(T, E, K_TOP, 1.1, 4, synth.S_ROUTE)
    return x, ids, w


def test_pack_of_288_expert_projections_bit_exact(layer):
    # the load-time pack of all 288 experts x 3 projections: codes, scale bytes and
    # scale_2 of every tensor equal the oracle's
    _, packed, ref = layer
    for p in PROJ:
        c, s, s2 = ref[p]
        ct, st = tile32(c, s)
        g = packed[p]
        assert np.array_equal(g.codes.cpu().numpy(), ct), f"pack codes differ: {p}"
        assert np.array_equal(g.scales.cpu().numpy(), st), f"pack scales differ: {p}"
        assert np.array_equal(g.scale_2.cpu().numpy().view(np.uint32), s2.view(np.uint32)), f"scale_2 differ: {p}"


@pytest.mark.parametrize("T,kernels", [
    (1, ("tiny", "tiny")),                        # 8 slots: gate/up routing itself, down with the combine
    (3, ("tiny", "tiny")),                        # 24 slots
    (4, ("decode_ksplit", "decode_resident")),    # 32 slots: 4-row tiles, gate/up K split over 4 waves
    (16, ("decode", "decode_resident")),          # 128 slots: 16-row tiles, H resident in LDS for down
    (64, ("decode", "decode_resident")),          # the benchmark's step
])
def test_decode_layer_every_token(layer, T, kernels):
    _, packed, ref = layer
    plan = nv.moe_plan(T, K_TOP, E, H, I, nv.LAYOUT_TILED32, nv.LAYOUT_TILED32)
    note(f"decode layer T={T}: {plan}")
    assert (plan["gate_up"], plan["down"]) == kernels and plan["fp16"]
    x, ids, w = _decode_inputs(T)
    y = bf16_host_f64(_moe(x, ids, w, packed))
    assert_close(y, _oracle_moe(x, ids, w, ref), f"decode T={T}")


def test_prefill_layer_every_token_permutation_and_chunks(layer):
    _, packed, ref = layer
    x, ids, w = _prefill_inputs()
    T = x.shape[0]
    plan = nv.moe_plan(T, K_TOP, E, H, I, nv.LAYOUT_TILED32, nv.LAYOUT_TILED32)
    note(f"prefill layer T=4096 Zipf: {plan}")
    assert (plan["gate_up"], plan["down"]) == ("prefill", "prefill")
    y = bf16_host_bits(_moe(x, ids, w, packed))
    # whole-batch properties: repeat, token permutation and the pinned prefill class are bitwise
    assert np.array_equal(bf16_host_bits(_moe(x, ids, w, packed)), y)
    p = np.random.default_rng(9).permutation(T)
    assert np.array_equal(bf16_host_bits(_moe(x[p], ids[p], w[p], packed)), y[p])
    assert np.array_equal(bf16_host_bits(_moe(x, ids, w, packed, kernel_class=nv.CLASS_PREFILL)), y)
    # the prompt in chunks with the prefill class pinned gives every token the same bits
    # (the last split ends on a 96-token chunk that the automatic choice would run on
    # decode tiles)
    for cuts in ([1024, 2048, 3072], [2048], [1000, 4000]):
        parts = []
        for a, b in zip([0] + cuts, cuts + [T]):
            parts.append(bf16_host_bits(_moe(x[a:b], ids[a:b], w[a:b], packed, kernel_class=nv.CLASS_PREFILL)))
        assert np.array_equal(np.concatenate(parts), y), f"chunks at {cuts}"
    note("prefill layer: oracle over all 4096 tokens")
    yf = bf16_host_f64(torch.from_numpy(y.view(np.int16)).view(torch.bfloat16))
    assert_close(yf, _oracle_moe(x, ids, w, ref), "prefill")


def test_decode_class_chunks_bitwise(layer):
    # a 64-token decode batch in chunks of 1, 15 and 48 tokens with the decode class
    # pinned equals the whole batch (the one-token chunk would take the K-split
    # kernel under the automatic choice)
    _, packed, _ = layer
    x, ids, w = _decode_inputs(64)
    whole = bf16_host_bits(_moe(x, ids, w, packed, kernel_class=nv.CLASS_DECODE))
    assert np.array_equal(whole, bf16_host_bits(_moe(x, ids, w, packed)))   # AUTO picks decode at 64 tokens
    parts = [bf16_host_bits(_moe(x[a:b], ids[a:b], w[a:b], packed, kernel_class=nv.CLASS_DECODE))
             for a, b in ((0, 1), (1, 16), (16, 64))]
    assert np.array_equal(np.concatenate(parts), whole)


def test_dense_mlp_every_row():
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
    note("dense MLP: oracle over all 2048 rows")
    h_ref = OM.linear_gated(x, res["gate"], res["up"])
    assert_close(bf16_host_f64(h), h_ref, "dense gated")
    y_ref = OM.dense_mlp(x, res["gate"], res["up"], res["down"])
    assert_close(bf16_host_f64(y), y_ref, "dense MLP")


@pytest.mark.parametrize("T", [64, 4096])
def test_w4a4_layer_every_token(layer, T):
    _, packed, ref = layer
    note(f"W4A4 layer T={T}")
    x, ids, w = _prefill_inputs() if T == 4096 else _decode_inputs(T)
    y = bf16_host_f64(_moe(x, ids, w, packed, W4A4_SCALES))
    assert_close(y, _oracle_moe(x, ids, w, ref, W4A4_SCALES), f"w4a4 T={T}")
