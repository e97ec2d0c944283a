"""GPU parity of every entry point against the CPU oracle, at sizes the oracle
finishes in seconds (several tiles and ragged tails), plus the edge cases.

Bit-exact: dequantized weights, packed codes/scales/scale_2, the permutation,
and the integer-exact linear. Within max|diff| <= 1e-2*max|ref| and cosine >=
0.9999: every bf16 output of a contraction."""
import concurrent.futures as cf
import json
import os

import numpy as np
import pytest
import torch

import nvfp4_moe_expert_amd as nv
import synth
from gpu_util import DEV, assert_close, bf16_dev, bf16_host_bits, bf16_host_f64, note, tile32, weight_dev
from oracle import formats as F
from oracle import mlp as OM
from oracle import nvfp4 as ONV

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ dequant
def _all_pairs():
    """Row r uses scale byte r in every block; every block holds the 16 codes in order."""
    n, k = 256, 64
    codes4 = np.tile(np.arange(16, dtype=np.uint8), (n, k // 16))
    codes = (codes4[:, 0::2] | (codes4[:, 1::2] << 4)).astype(np.uint8)
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], k // 16, axis=1)
    return codes, scales


@pytest.mark.parametrize("s2", [1.0, float(np.float32(1.0) / np.float32(2688.0)), 3.7e-5, 0.0])
def test_dequant_all_code_scale_pairs_bit_exact(s2):
    note(f"dequant all pairs s2={s2}")
    codes, scales = _all_pairs()
    w = weight_dev((codes[None], scales[None], np.float32(s2)))
    u, s = nv.dequant(w)
    torch.cuda.synchronize()
    ref_u, ref_s = ONV.dequant(codes, scales, np.float32(s2))
    gu = F.bf16_to_f32(bf16_host_bits(u[0]))
    gs = s[0].cpu().numpy()
    finite = np.isfinite(ref_u)
    assert np.array_equal(np.isnan(gu), ~finite) and np.array_equal(np.isnan(gs), ~np.isfinite(ref_s))
    assert np.array_equal(gu[finite].view(np.uint32), ref_u[finite].view(np.uint32))
    fs = np.isfinite(ref_s)
    assert np.array_equal(gs[fs].view(np.uint32), ref_s[fs].view(np.uint32))


def test_dequant_only_one_output():
    codes, scales = _all_pairs()
    w = weight_dev((codes[None], scales[None], np.float32(2.0)))
    u, s = nv.dequant(w, unscaled=True, scaled=False)
    assert s is None and u is not None
    u2, s2 = nv.dequant(w, unscaled=False, scaled=True)
    assert u2 is None
    ref_u, ref_s = ONV.dequant(codes, scales, np.float32(2.0))
    f = np.isfinite(ref_s)
    assert np.array_equal(s2[0].cpu().numpy()[f].view(np.uint32), ref_s[f].view(np.uint32))


# ------------------------------------------------------------------ pack
def _golden():
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pack_small.json")))
    w = np.zeros(g["w_bf16"]["shape"], np.uint16)
    for r, c, h in g["w_bf16"]["nonzero"]:
        w[r, c] = int(h, 16)
    return w[None]


def _pack_cases():
    rng = np.random.default_rng(77)
    cases = {
        "golden": _golden(),
        "normal_0.02": np.stack([synth.bf16_normal((64, 256), 0.02, 30, i) for i in range(3)]),
        "normal_1_ragged_rows": np.stack([synth.bf16_normal((33, 512), 1.0, 31, i) for i in range(2)]),
        "single_block": synth.bf16_normal((1, 32), 0.5, 32)[None],
        "mixed_magnitude": synth.f32_to_bf16_bits(
            (rng.standard_normal((24, 256)) * np.exp2(rng.integers(-20, 6, (24, 1)))).astype(np.float32))[None],
        "cauchy": synth.f32_to_bf16_bits((rng.standard_cauchy((24, 256)) * 0.01).astype(np.float32))[None],
        "expert_sized": np.stack([synth.bf16_normal((1536, 4096), 0.02, 33, i) for i in range(2)]),
    }
    z = np.zeros((3, 8, 64), np.uint16)
    z[1] = synth.bf16_normal((8, 64), 0.02, 34)
    z[1, :, 16:32] = 0
    z[1, 3, :] = 0x8000
    z[2] = synth.bf16_normal((8, 64), 0.02, 35)
    z[2, 0, 1] = 0x8000
    cases["zeros_and_negzeros"] = z
    t = np.zeros((2, 2, 32), np.uint16)
    t[0, 0, 0] = 0x0001
    t[1, 1, 0] = 0x3F80
    t[1, 1, 16] = 0x3780
    cases["subnormal"] = t
    return cases


@pytest.mark.parametrize("name", list(_pack_cases()))
def test_pack_bit_exact(name):
    w = _pack_cases()[name]
    note(f"pack {name} {w.shape}")
    g = nv.pack(bf16_dev(w))
    torch.cuda.synchronize()
    c, s, s2 = ONV.pack_batch(w)
    assert np.array_equal(g.codes.cpu().numpy(), c)
    assert np.array_equal(g.scales.cpu().numpy(), s)
    assert np.array_equal(g.scale_2.cpu().numpy().view(np.uint32), s2.view(np.uint32))


def test_fp4_convert_equals_e2m1_rounding_everywhere():
    # the pack encodes e2m1 with the device's fp4 convert: it must round every fp32
    # input (both signs, 2^32 patterns, NaNs skipped) as the nearest-even reading does
    note("fp4 convert self-test over all fp32 bit patterns")
    assert nv.selftest_fp4_convert(DEV) == 0


def test_pack_2d_input_and_repeat_determinism():
    w = synth.bf16_normal((48, 128), 0.02, 36)
    a = nv.pack(bf16_dev(w))
    b = nv.pack(bf16_dev(w))
    assert torch.equal(a.codes, b.codes) and torch.equal(a.scales, b.scales)
    assert a.codes.shape == (1, 48, 64)


# ------------------------------------------------------------------ route
def _route_cases():
    r = np.random.default_rng(5)
    cases = []
    ids, _ = synth.topk_softmax_routing(8, 16, 4, 2, synth.S_ROUTE)
    cases.append(("cfg2", ids, 16, 0))
    for T in (1, 16, 64):
        ids, _ = synth.topk_softmax_routing(T, 288, 8, 3, synth.S_ROUTE, T)
        cases.append((f"decode_T{T}", ids, 288, 0))
    ids, _ = synth.zipf_routing(4096, 288, 8, 1.1, 4, synth.S_ROUTE)
    cases.append(("prefill_zipf", ids, 288, 0))
    cases.append(("skipped_ep", r.integers(0, 30, (37, 3)).astype(np.int32), 5, 10))
    cases.append(("one_expert", np.zeros((100, 2), np.int32), 1, 0))
    cases.append(("many_experts", r.integers(0, 4096, (50, 8)).astype(np.int32), 4096, 0))
    dup = r.integers(0, 6, (70, 4)).astype(np.int32)
    dup[:, 1] = dup[:, 0]
    cases.append(("duplicates", dup, 6, 0))
    cases.append(("all_skipped", r.integers(0, 16, (9, 4)).astype(np.int32), 16, 1000))
    cases.append(("ragged_S", r.integers(0, 3, (67, 1)).astype(np.int32), 3, 0))
    cases.append(("negative_ids", r.integers(-5, 5, (20, 2)).astype(np.int32), 5, 0))
    # prefill-sized batches with uniform ids, one of them ragged and with skipped ids
    cases.append(("uniform_4096", r.integers(0, 288, (4096, 8)).astype(np.int32), 288, 0))
    cases.append(("uniform_4097_skips", r.integers(0, 300, (4097, 8)).astype(np.int32), 288, 6))
    # 4096 experts over several windows; 63 windows of 2112 slots (the most windows: 64)
    cases.append(("many_experts_large", r.integers(0, 4096, (1000, 8)).astype(np.int32), 4096, 0))
    cases.append(("windows_63", r.integers(-3, 290, (16500, 8)).astype(np.int32), 288, 0))
    return cases


@pytest.mark.parametrize("ci", range(len(_route_cases())))
def test_route_bit_exact(ci):
    name, ids, E, eb = _route_cases()[ci]
    note(f"route {name} ids{ids.shape} E={E} eb={eb}")
    off, perm, inv = nv.moe_route(torch.from_numpy(ids).to(DEV), E, eb)
    torch.cuda.synchronize()
    counts, roff, rperm, rinv = OM.route(ids, E, eb)
    assert np.array_equal(off.cpu().numpy(), roff)
    V = int(roff[-1])
    assert np.array_equal(perm.cpu().numpy()[:V], rperm)
    assert np.array_equal(inv.cpu().numpy(), rinv)


@pytest.mark.parametrize("name", ["prefill_zipf", "uniform_4097_skips", "many_experts_large", "windows_63"])
def test_route_one_workgroup_large_batch(name):
    # without scratch one workgroup routes a batch the scratch path spreads over windows
    _, ids, E, eb = next(c for c in _route_cases() if c[0] == name)
    note(f"route (no scratch) {name} ids{ids.shape} E={E} eb={eb}")
    assert nv.load_library().nvfp4_moe_route_workspace_size(ids.shape[0], ids.shape[1], E) > 0
    off, perm, inv = nv.moe_route(torch.from_numpy(ids).to(DEV), E, eb, scratch=False)
    torch.cuda.synchronize()
    counts, roff, rperm, rinv = OM.route(ids, E, eb)
    assert np.array_equal(off.cpu().numpy(), roff)
    assert np.array_equal(perm.cpu().numpy()[:int(roff[-1])], rperm)
    assert np.array_equal(inv.cpu().numpy(), rinv)


def test_route_unaligned_ids():
    # ids that do not start on a 16-byte boundary
    r = np.random.default_rng(11)
    ids = r.integers(0, 40, (1 + 33 * 5,)).astype(np.int32)
    dev = torch.from_numpy(ids).to(DEV)[1:].view(33, 5)
    assert dev.data_ptr() % 16 != 0
    off, perm, inv = nv.moe_route(dev, 40, 0)
    torch.cuda.synchronize()
    counts, roff, rperm, rinv = OM.route(ids[1:].reshape(33, 5), 40, 0)
    assert np.array_equal(off.cpu().numpy(), roff)
    assert np.array_equal(perm.cpu().numpy()[:int(roff[-1])], rperm)
    assert np.array_equal(inv.cpu().numpy(), rinv)


def test_route_empty_batch():
    ids = torch.zeros((0, 8), dtype=torch.int32, device=DEV)
    off, perm, inv = nv.moe_route(ids, 16, 0)
    torch.cuda.synchronize()
    assert np.all(off.cpu().numpy() == 0)


# ------------------------------------------------------------------ linear
@pytest.mark.parametrize("M,N,K,seed", [
    (4, 256, 512, 1),        # single NVFP4 linear workload: X[4,512], W[256,512]
    (16, 80, 4096, 49), (3, 48, 1536, 51),   # N % 64 != 0, row-major: the fallback GEMM
    (7, 64, 2048, 50),                        # at most 16 rows: the decode kernel
    (1, 64, 32, 40), (16, 128, 256, 41), (17, 100, 96, 42), (130, 48, 160, 43),
    (300, 256, 1024, 44), (129, 200, 544, 45),
    (4000, 8192, 256, 46),   # prefill tiles, full-width workgroups (grid of 32 x 16), ragged last tile
    (12, 128, 192, 133), (5, 64, 384, 134),   # at most 16 rows, K % 256 != 0: 128-input decode stages
    (40, 96, 192, 135), (300, 64, 1088, 136),  # more rows, K % 256 != 0: prefill tiles, last stage partial
    (40, 96, 160, 141),                        # K % 64 == 32: the fallback
])
def test_linear_vs_oracle(M, N, K, seed):
    note(f"linear M={M} N={N} K={K}")
    x = synth.bf16_normal((M, K), 1.0, seed, synth.S_X)
    wp = ONV.pack(synth.bf16_normal((N, K), 0.02, seed, synth.S_W))
    y = nv.linear(bf16_dev(x), weight_dev(wp))
    torch.cuda.synchronize()
    assert_close(bf16_host_f64(y), OM.linear(x, wp), f"linear {M}x{N}x{K}")


@pytest.mark.parametrize("M", [4, 40])
def test_linear_integer_exact(M):
    # scale bytes 1.0, scale_2 1.0, integer activations: every partial sum is exact in
    # fp32, so the bf16 output must be the nearest-even rounding of the exact result
    N, K = 64, 512
    g = np.random.default_rng(M)
    x = synth.bf16_integers((M, K), -8, 8, 46, M)
    codes4 = g.integers(0, 16, (N, K)).astype(np.uint8)
    codes = (codes4[:, 0::2] | (codes4[:, 1::2] << 4)).astype(np.uint8)
    scales = np.full((N, K // 16), 0x38, np.uint8)
    wp = (codes, scales, np.float32(1.0))
    y = nv.linear(bf16_dev(x), weight_dev(wp))
    exact = OM.linear(x, wp)
    assert np.array_equal(bf16_host_bits(y), F.f32_to_bf16(exact.astype(np.float32)))


def test_linear_empty_rows():
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV)
    wp = ONV.pack(synth.bf16_normal((32, 64), 0.02, 47))
    y = nv.linear(x, weight_dev(wp))
    assert y.shape == (0, 32)


@pytest.mark.parametrize("M,N,K", [(4, 128, 512), (33, 96, 256), (200, 64, 128), (5, 48, 2048), (16, 32, 4096)])
def test_linear_gated_vs_oracle(M, N, K):
    note(f"linear_gated M={M} N={N} K={K}")
    x = synth.bf16_normal((M, K), 1.0, 48, M)
    wg = ONV.pack(synth.bf16_normal((N, K), 0.05, 48, synth.S_GATE, M))
    wu = ONV.pack(synth.bf16_normal((N, K), 0.05, 48, synth.S_UP, M))
    h = nv.linear_gated(bf16_dev(x), weight_dev(wg), weight_dev(wu))
    torch.cuda.synchronize()
    assert_close(bf16_host_f64(h), OM.linear_gated(x, wg, wu), "linear_gated")


# ------------------------------------------------------------------ moe
def _pack_experts(E, N, K, sigma, seed, stream):
    """Oracle packs of E seeded bf16 experts [N, K], packed on threads (numpy releases
    the GIL); the same result as ONV.pack_batch."""
    wb = synth.expert_weights(E, N, K, sigma, seed, stream)
    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        outs = list(ex.map(ONV.pack, wb))
    return (np.stack([o[0] for o in outs]), np.stack([o[1] for o in outs]),
            np.array([o[2] for o in outs], dtype=np.float32))


def _moe_problem(T, k, E, H, I, seed, sigma=0.02, ids=None, weights=None):
    x = synth.bf16_normal((T, H), 1.0, seed, synth.S_X)
    if ids is None:
        ids, weights = synth.topk_softmax_routing(T, E, k, seed, synth.S_ROUTE)
    gate = _pack_experts(E, I, H, sigma, seed, synth.S_GATE)
    up = _pack_experts(E, I, H, sigma, seed, synth.S_UP)
    down = _pack_experts(E, H, I, sigma, seed, synth.S_DOWN)
    return x, ids.astype(np.int32), weights.astype(np.float32), gate, up, down


def _run_moe(x, ids, w, gate, up, down, eb=0, layout=nv.LAYOUT_ROWS, kernel_class=None):
    return nv.moe_grouped(bf16_dev(x), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV),
                          weight_dev(gate, layout), weight_dev(up, layout), weight_dev(down, layout), expert_begin=eb,
                          kernel_class=kernel_class)


# Every case names the kernels it reaches (nvfp4_moe_plan, checked before the run):
# gate/up kernel, down kernel and the down kernel's width (64-row blocks per wave
# stream of the resident-H decode kernel; 32-row weight blocks per wave of the
# prefill kernel). Widths of the decode down kernel follow the compute-unit count
# (256 on MI355X).
KS, DEC, RES, PRE, FB, TY = "decode_ksplit", "decode", "decode_resident", "prefill", "fallback", "tiny"


@pytest.mark.parametrize("T,k,E,H,I,seed,layout,kern", [
    # grouped decode MoE workload: 16 experts, top-4, 8 tokens (32 slots: 4-row tiles)
    (8, 4, 16, 2048, 512, 2, 0, (KS, RES, 1)),
    (6, 2, 4, 2048, 1536, 70, 0, (KS, RES, 1)),      # K-split gate/up K=2048, resident down K=1536
    (3, 2, 2, 4096, 512, 71, 0, (TY, TY, 0)),        # 3 tokens: the two-launch path, K=4096 (two stages per wave)
    # at most 4 tokens: gate/up routing itself on 4-row tiles, down with the combine
    (1, 8, 16, 4096, 1536, 141, 1, (TY, TY, 0)),     # the model's shapes, one token
    (2, 8, 16, 4096, 1536, 142, 0, (TY, TY, 0)),     # 16 slots: four per down wave
    (3, 8, 12, 2048, 2048, 143, 1, (TY, TY, 0)),     # 24 slots over 12 experts (multi-row tiles), down 4 stages
    (4, 8, 12, 2048, 2048, 148, 1, (KS, RES, 1)),    # 32 slots: the K-split gate/up
    (3, 4, 6, 512, 512, 144, 0, (TY, TY, 0)),        # one stage each: waves 1..3 of gate/up idle
    (3, 8, 8, 2560, 1024, 145, 0, (TY, TY, 0)),      # gate/up 5 stages (waves with one and two), down 2
    (1, 24, 40, 1024, 512, 149, 1, (TY, TY, 0)),     # top-24: eight slots per down wave
    (1, 16, 300, 1024, 512, 146, 1, (TY, TY, 0)),    # top-16 over 300 experts: four slots per down wave
    (32, 1, 2, 2048, 512, 72, 0, (KS, RES, 1)),      # 32 slots, 16 per expert: K-split on 4-row tiles
    (40, 2, 3, 512, 2048, 73, 0, (PRE, PRE, 1)),     # 80 slots over 3 experts: prefill tiles
    # decode tiles (more than 32 slots, at most 16 rows per local expert on average)
    (16, 4, 16, 4096, 1536, 120, 1, (DEC, RES, 1)),  # gate/up decode kernel K=4096, down K=1536 one block per wave
    (16, 4, 16, 2048, 1536, 121, 1, (DEC, RES, 1)),  # gate/up decode kernel K=2048
    (64, 4, 32, 4096, 512, 122, 1, (DEC, RES, 2)),   # 48-tile bound x 4096 rows: two 64-row blocks per wave
    (128, 4, 32, 4096, 512, 123, 1, (DEC, RES, 4)),  # 64-tile bound: four 64-row blocks per wave
    (64, 4, 32, 4096, 512, 124, 0, (DEC, RES, 2)),   # the same on row-major weights
    (12, 4, 16, 4096, 2560, 125, 1, (DEC, DEC, 0)),  # down K=2560 > 2048: the streaming decode kernel
    (600, 8, 320, 512, 512, 151, 1, (DEC, RES, 4)),  # 4800 slots: the windowed route feeding decode tiles
    # tensor-parallel shards of the intermediate size (row-major: K % 256 != 0)
    (16, 4, 16, 4096, 384, 130, 0, (DEC, DEC, 0)),   # I/4 = 384: down K=384 in 128-input stages
    (16, 4, 16, 4096, 192, 131, 0, (DEC, DEC, 0)),   # I/8 = 192: the last stage half masked
    (3, 2, 4, 4096, 192, 132, 0, (KS, DEC, 0)),      # 6 slots: K-split gate/up, down K=192
    (5, 2, 3, 64, 32, 60, 0, (FB, FB, 0)),           # shapes only the fallback covers
    (1, 8, 12, 256, 96, 61, 0, (FB, FB, 0)),
    (200, 2, 4, 128, 64, 62, 0, (PRE, PRE, 1)),      # 100 rows per expert; K = 128 and 64: one partial stage each
    (64, 8, 20, 256, 160, 63, 0, (PRE, FB, 0)),      # prefill gate/up (bf16 form), down K = 160 on the fallback
    # prefill tiles
    (300, 4, 6, 512, 256, 74, 0, (PRE, PRE, 1)),     # fp16 gate/up, 2 tiles per expert (full + ragged)
    (150, 8, 40, 256, 512, 75, 0, (PRE, PRE, 1)),    # ~30 rows per expert (1-row-block tiles, two stages ahead)
    (600, 2, 8, 512, 256, 76, 0, (PRE, PRE, 1)),     # two activation rows per prep workgroup (ragged last one)
    (600, 8, 16, 256, 256, 77, 0, (PRE, PRE, 1)),    # 4800 slots: the route's three windows
    (300, 4, 6, 768, 1280, 126, 1, (PRE, PRE, 1)),   # odd stage counts: gate/up 3, down 5 (3- and 4-block tiles)
    (150, 8, 40, 768, 1280, 127, 1, (PRE, PRE, 1)),  # odd stage counts on 1- and 2-block tiles (two ahead)
    (2048, 8, 16, 2048, 768, 128, 1, (PRE, PRE, 2)), # down 3 stages on full-width (512-row) workgroups
    # prefill tiles on row-major weights whose K ends on a partial 256-input stage
    (200, 4, 8, 1088, 320, 137, 0, (PRE, PRE, 1)),   # gate/up K = 4 stages + 64, down K = 256 + 64
    (200, 4, 8, 1056, 288, 140, 0, (FB, FB, 0)),     # K % 64 == 32 (odd scale row pitch): the fallback
    (300, 4, 6, 4096, 384, 138, 0, (PRE, PRE, 1)),   # tensor-parallel shard I/4: down K = 384
    (300, 4, 6, 512, 192, 139, 0, (PRE, PRE, 1)),    # tensor-parallel shard I/8: down K = 192
])
def test_moe_vs_oracle(T, k, E, H, I, seed, layout, kern):
    plan = nv.moe_plan(T, k, E, H, I, layout, layout)
    note(f"moe T={T} k={k} E={E} H={H} I={I} layout={layout}: {plan}")
    assert (plan["gate_up"], plan["down"], plan["down_width"]) == kern
    x, ids, w, gate, up, down = _moe_problem(T, k, E, H, I, seed, sigma=0.05)
    y = _run_moe(x, ids, w, gate, up, down, layout=layout)
    torch.cuda.synchronize()
    assert_close(bf16_host_f64(y), OM.moe(x, ids, w, gate, up, down), "moe")


@pytest.mark.parametrize("cls,T,k,E,H,I,cuts", [
    (nv.CLASS_PREFILL, 600, 8, 16, 512, 256, [1, 100, 340]),   # chunks of 1, 99, 240 and 260 tokens
    (nv.CLASS_DECODE, 96, 4, 32, 512, 512, [1, 9, 40]),        # a one-token chunk would take the K-split
    (nv.CLASS_DECODE, 600, 8, 16, 512, 512, [1, 100, 340]),    # ~300 rows per expert in 16-row tiles, 4800 slots
])
def test_moe_pinned_class_chunks_bitwise(cls, T, k, E, H, I, cuts):
    # a pinned kernel class gives every token the same bits whatever the chunking
    # (TensorFold #308, "Questions", item 4), and stays within the oracle's bar
    note(f"moe class {cls} T={T} chunks at {cuts}")
    x, ids, w, gate, up, down = _moe_problem(T, k, E, H, I, 129 + cls, sigma=0.05)
    whole = bf16_host_bits(_run_moe(x, ids, w, gate, up, down, layout=1, kernel_class=cls))
    parts = [bf16_host_bits(_run_moe(x[a:b], ids[a:b], w[a:b], gate, up, down, layout=1, kernel_class=cls))
             for a, b in zip([0] + cuts, cuts + [T])]
    assert np.array_equal(np.concatenate(parts), whole)
    yf = bf16_host_f64(torch.from_numpy(whole.view(np.int16)).view(torch.bfloat16))
    assert_close(yf, OM.moe(x, ids, w, gate, up, down), "moe pinned class")


def test_moe_expert_parallel_slice_and_duplicates():
    T, k, E, H, I = 30, 4, 4, 128, 64
    g = np.random.default_rng(3)
    ids = g.integers(0, 12, (T, k)).astype(np.int32)
    ids[:, 1] = ids[:, 0]                          # duplicate ids count twice
    w = g.uniform(0.1, 1.0, (T, k)).astype(np.float32)
    x, _, _, gate, up, down = _moe_problem(T, k, E, H, I, 64, sigma=0.05, ids=ids, weights=w)
    y = _run_moe(x, ids, w, gate, up, down, eb=4)
    torch.cuda.synchronize()
    ref = OM.moe(x, ids, w, gate, up, down, expert_begin=4)
    assert_close(bf16_host_f64(y), ref, "moe ep slice")
    none_local = ~np.any((ids >= 4) & (ids < 8), axis=1)
    assert np.all(bf16_host_f64(y)[none_local] == 0)


@pytest.mark.parametrize("case", ["ep_slice", "one_expert", "no_local_token"])
def test_moe_tiny_routing_edges(case):
    # the two-launch path derives its tiles from the ids in every workgroup:
    # ids outside this GPU's experts, duplicates within a token, all 24 slots on
    # one expert (tiles of 16 and 8 slots of one expert), and a token with no local slot
    T, k, E, H, I = 3, 8, 16, 1024, 512
    g = np.random.default_rng(147)
    if case == "ep_slice":
        ids = g.integers(0, 48, (T, k)).astype(np.int32)
        ids[:, 1] = ids[:, 0]
        eb = 16
    elif case == "one_expert":
        ids = np.full((T, k), 21, np.int32)
        eb = 16
    else:
        ids = g.integers(16, 32, (T, k)).astype(np.int32)
        ids[2] = g.integers(40, 60, k)
        eb = 16
    w = g.uniform(0.1, 1.0, (T, k)).astype(np.float32)
    plan = nv.moe_plan(T, k, E, H, I, 0, 0)
    assert (plan["gate_up"], plan["down"]) == (TY, TY)
    x, _, _, gate, up, down = _moe_problem(T, k, E, H, I, 147, sigma=0.05, ids=ids, weights=w)
    note(f"moe tiny edges {case}: ids {ids.tolist()}")
    y = _run_moe(x, ids, w, gate, up, down, eb=eb)
    torch.cuda.synchronize()
    ref = OM.moe(x, ids, w, gate, up, down, expert_begin=eb)
    assert_close(bf16_host_f64(y), ref, f"moe tiny {case}")
    none_local = ~np.any((ids >= eb) & (ids < eb + E), axis=1)
    assert np.all(bf16_host_f64(y)[none_local] == 0)


def test_moe_all_slots_skipped_gives_zero():
    x, ids, w, gate, up, down = _moe_problem(9, 4, 4, 64, 32, 65)
    y = _run_moe(x, ids, w, gate, up, down, eb=100)
    torch.cuda.synchronize()
    assert np.all(bf16_host_bits(y) == 0)


def test_moe_empty_batch():
    _, _, _, gate, up, down = _moe_problem(1, 2, 3, 64, 32, 66)
    y = nv.moe_grouped(torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV),
                       torch.zeros((0, 2), dtype=torch.int32, device=DEV),
                       torch.zeros((0, 2), dtype=torch.float32, device=DEV),
                       weight_dev(gate), weight_dev(up), weight_dev(down))
    assert y.shape == (0, 64)


@pytest.mark.parametrize("T,k,E,H,I", [(8, 4, 16, 2048, 512), (200, 2, 4, 128, 64), (3, 8, 16, 4096, 1536)])
def test_moe_token_permutation_and_repeat_bitwise(T, k, E, H, I):
    x, ids, w, gate, up, down = _moe_problem(T, k, E, H, I, 67, sigma=0.05)
    y1 = bf16_host_bits(_run_moe(x, ids, w, gate, up, down))
    y2 = bf16_host_bits(_run_moe(x, ids, w, gate, up, down))
    assert np.array_equal(y1, y2)
    p = np.random.default_rng(1).permutation(T)
    yp = bf16_host_bits(_run_moe(x[p], ids[p], w[p], gate, up, down))
    assert np.array_equal(yp, y1[p])


@pytest.mark.parametrize("T,k,E,H,I", [(1, 8, 12, 4096, 512),     # one token: the two-launch path
                                       (8, 4, 16, 2048, 512),     # decode tiles
                                       (300, 4, 6, 512, 256),     # prefill tiles, fp16 form
                                       (600, 8, 16, 256, 256)])   # 4800 slots: three-launch route
def test_moe_graph_capture_replays_equal_eager(T, k, E, H, I):
    # the library allocates, synchronizes and clears nothing on the host side, so a
    # captured call replays; every replay, with eager work and synchronizations in
    # between, must give the eager result bit for bit
    note(f"moe graph capture T={T} k={k} E={E} H={H} I={I}")
    x, ids, w, gate, up, down = _moe_problem(T, k, E, H, I, 78, sigma=0.05)
    xd, idd, wd = bf16_dev(x), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV)
    gw, uw, dw = weight_dev(gate), weight_dev(up), weight_dev(down)
    ws = torch.empty((nv.moe_workspace_size(T, k, E, H, I),), dtype=torch.uint8, device=DEV)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    nv.moe_grouped(xd, idd, wd, gw, uw, dw, workspace=ws, out=out)
    torch.cuda.synchronize()
    eager = out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        nv.moe_grouped(xd, idd, wd, gw, uw, dw, workspace=ws, out=out)   # warm-up on the side stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        nv.moe_grouped(xd, idd, wd, gw, uw, dw, workspace=ws, out=out)
    for rep in range(3):
        out.zero_()
        ws.fill_(0x5A)                                                     # stale workspace contents
        _ = _run_moe(x[::-1].copy(), ids[::-1].copy(), w[::-1].copy(), gate, up, down)   # eager work between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"


def test_pack_and_linear_graph_capture_replays_equal_eager():
    # pack (both quantize kernels' layouts) and the dense linear paths captured in one graph
    note("pack + linear graph capture")
    wb = synth.bf16_normal((3, 256, 512), 0.02, 79)
    wd = torch.from_numpy(wb.view(np.int16)).view(torch.bfloat16).to(DEV)
    xs = [bf16_dev(synth.bf16_normal((m, 512), 1.0, 80, m)) for m in (4, 300)]
    lin = ONV.pack(wb[0])
    lw = weight_dev((lin[0][None], lin[1][None], np.float32(lin[2])))
    outs = [torch.empty((x.shape[0], 256), dtype=torch.bfloat16, device=DEV) for x in xs]

    def work():
        p = [nv.pack(wd, layout=nv.LAYOUT_TILED32), nv.pack(wd, layout=nv.LAYOUT_ROWS)]
        for x, o in zip(xs, outs):
            nv.linear(x, lw, out=o)
        return p

    eager_p = work()
    torch.cuda.synchronize()
    eager_o = [o.clone() for o in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        work()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap_p = work()
    for rep in range(3):
        for o in outs:
            o.zero_()
        for pk in cap_p:
            pk.codes.zero_()
            pk.scales.zero_()
        work()                                                             # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(cap_p, eager_p):
            assert torch.equal(a.codes, b.codes) and torch.equal(a.scales, b.scales), f"pack, replay {rep}"
            assert torch.equal(a.scale_2, b.scale_2), f"scale_2, replay {rep}"
        for a, b in zip(outs, eager_o):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"linear, replay {rep}"


@pytest.mark.parametrize("T,I", [(24, 128), (200, 256)])
def test_moe_k1_matches_dense_mlp_path(T, I):
    # one expert per token with weight 1: the grouped path equals linear_gated then
    # linear up to summation order and the fp16 form (the two entry points may use
    # different kernels)
    E, H = 3, 256
    ids = np.full((T, 1), 1, np.int32)
    w = np.ones((T, 1), np.float32)
    x, _, _, gate, up, down = _moe_problem(T, 1, E, H, I, 68, sigma=0.05, ids=ids, weights=w)
    y = _run_moe(x, ids, w, gate, up, down)
    gd, ud, dd = weight_dev(gate).expert(1), weight_dev(up).expert(1), weight_dev(down).expert(1)
    h = nv.linear_gated(bf16_dev(x), gd, ud)
    y2 = nv.linear(h, dd)
    torch.cuda.synchronize()
    assert_close(bf16_host_f64(y), bf16_host_f64(y2), "moe k=1 vs dense path")


@pytest.mark.parametrize("T,k,E,H,I", [(8, 4, 16, 256, 128), (2, 8, 16, 1024, 512)])
def test_moe_timed_events_same_result(T, k, E, H, I):
    x, ids, w, gate, up, down = _moe_problem(T, k, E, H, I, 69, sigma=0.05)
    y1 = bf16_host_bits(_run_moe(x, ids, w, gate, up, down))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    y2 = nv.moe_grouped(bf16_dev(x), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV),
                        weight_dev(gate), weight_dev(up), weight_dev(down), events=ev)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_host_bits(y2), y1)
    times = [ev[i].elapsed_time(ev[i + 1]) for i in range(4)]
    assert all(t >= 0 for t in times)


# ------------------------------------------------------------------ tiled layout
TILED = nv.LAYOUT_TILED32


def test_pack_tiled_bit_exact_and_relayout_roundtrip():
    w = synth.bf16_normal((3, 96, 512), 0.03, 80)
    note("pack tiled (3, 96, 512)")
    gt = nv.pack(bf16_dev(w), layout=TILED)
    gr = nv.pack(bf16_dev(w))
    back = nv.relayout(gt, nv.LAYOUT_ROWS)
    fwd = nv.relayout(gr, TILED)
    torch.cuda.synchronize()
    c, s, s2 = ONV.pack_batch(w)
    ct, st = tile32(c, s)
    assert np.array_equal(gt.codes.cpu().numpy(), ct)
    assert np.array_equal(gt.scales.cpu().numpy(), st)
    assert np.array_equal(gt.scale_2.cpu().numpy().view(np.uint32), s2.view(np.uint32))
    assert torch.equal(fwd.codes, gt.codes) and torch.equal(fwd.scales, gt.scales)
    assert torch.equal(back.codes, gr.codes) and torch.equal(back.scales, gr.scales)


def test_dequant_tiled_matches_rows():
    w = ONV.pack_batch(synth.bf16_normal((2, 64, 256), 0.05, 81))
    ur, sr = nv.dequant(weight_dev(w))
    ut, stl = nv.dequant(weight_dev(w, TILED))
    torch.cuda.synchronize()
    assert torch.equal(ur.view(torch.int16), ut.view(torch.int16))
    assert torch.equal(sr.view(torch.int32), stl.view(torch.int32))


@pytest.mark.parametrize("M,N,K", [
    (4, 256, 512),       # decode kernel
    (16, 96, 256),       # n % 64 != 0: the prefill kernel takes tiled weights
    (300, 256, 1024),    # prefill, half-width workgroups
    (4000, 8192, 256),   # prefill, full-width workgroups
])
def test_linear_tiled_vs_oracle_and_rows(M, N, K):
    note(f"linear tiled M={M} N={N} K={K}")
    x = synth.bf16_normal((M, K), 1.0, 82, synth.S_X, M)
    w = ONV.pack(synth.bf16_normal((N, K), 0.02, 82, synth.S_W, M))
    yt = nv.linear(bf16_dev(x), weight_dev(w, TILED))
    yr = nv.linear(bf16_dev(x), weight_dev(w))
    torch.cuda.synchronize()
    assert_close(bf16_host_f64(yt), OM.linear(x, w), "linear tiled")
    if N % 64 == 0 or M > 16:       # same kernel for both layouts: same bits
        assert np.array_equal(bf16_host_bits(yt), bf16_host_bits(yr))


@pytest.mark.parametrize("T,k,E,H,I,seed", [
    (8, 4, 16, 2048, 512, 83),      # decode tiles
    (300, 4, 6, 512, 256, 84),      # prefill tiles, full and ragged
    (150, 8, 40, 256, 512, 85),     # prefill tiles, ~30 rows per expert
])
def test_moe_tiled_vs_oracle_and_rows(T, k, E, H, I, seed):
    note(f"moe tiled T={T} k={k} E={E} H={H} I={I}")
    x, ids, w, gate, up, down = _moe_problem(T, k, E, H, I, seed, sigma=0.05)
    args = (bf16_dev(x), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV))
    yt = nv.moe_grouped(*args, weight_dev(gate, TILED), weight_dev(up, TILED), weight_dev(down, TILED))
    yr = nv.moe_grouped(*args, weight_dev(gate), weight_dev(up), weight_dev(down))
    torch.cuda.synchronize()
    assert_close(bf16_host_f64(yt), OM.moe(x, ids, w, gate, up, down), "moe tiled")
    assert np.array_equal(bf16_host_bits(yt), bf16_host_bits(yr))


@pytest.mark.gpu
@pytest.mark.parametrize("T,k,E,H,I,seed", [
    (8, 4, 16, 2048, 512, 86),      # decode tiles
    (300, 4, 6, 512, 256, 87),      # prefill tiles, full and ragged
])
def test_moe_mixed_layouts_bitwise(T, k, E, H, I, seed):
    """gate and up share a layout; down may hold the other one. Each projection's
    kernel reads its own layout, so the output is bitwise that of all-tiled weights.
    A gate/up pair in two layouts is refused."""
    note(f"moe mixed layouts T={T} k={k} E={E} H={H} I={I}")
    x, ids, w, gate, up, down = _moe_problem(T, k, E, H, I, seed, sigma=0.05)
    args = (bf16_dev(x), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV))
    gt, ut, dt = weight_dev(gate, TILED), weight_dev(up, TILED), weight_dev(down, TILED)
    gr, ur, dr = weight_dev(gate), weight_dev(up), weight_dev(down)
    ref = bf16_host_bits(nv.moe_grouped(*args, gt, ut, dt))
    for g_, u_, d_ in ((gt, ut, dr), (gr, ur, dt)):
        y = nv.moe_grouped(*args, g_, u_, d_)
        torch.cuda.synchronize()
        assert np.array_equal(bf16_host_bits(y), ref)
    with pytest.raises(RuntimeError):
        nv.moe_grouped(*args, gt, ur, dt)

# ------------------------------------------------------------------ W4A4 activations
def _scale_dev(*v):
    return torch.tensor([np.float32(a) for a in v], dtype=torch.float32, device=DEV)


def _ties_block_rows():
    """Rows of 16-blocks with scale byte 0x38 (1.0) at input_scale 1/8: each block
    holds the max 6/8 and every e2m1 midpoint (0.25 .. 5.0)/8 with both signs, so
    every tie-to-even decision and -0 appear."""
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    blk = np.concatenate([[6.0], mids, -mids, [0.0]]).astype(np.float32) / 8    # 16 values
    row = np.tile(blk, 4)
    x = np.stack([row, -row, np.roll(row, 3)])
    bits = F.f32_to_bf16(x)
    bits[2, 5] = 0x8000          # -0 inside a nonzero block
    return bits


@pytest.mark.parametrize("case", ["typical", "saturating", "zero_scale", "h_rows", "ties"])
def test_quantize_act_bit_exact(case):
    note(f"quantize_act {case}")
    if case == "ties":
        x, s = _ties_block_rows(), 1.0 / 8
    else:
        rows, k, s, seed = {"typical": (37, 512, 4.0 / 2688, 90), "saturating": (8, 4096, 0.5 / 2688, 91),
                            "zero_scale": (5, 256, 0.0, 92), "h_rows": (300, 1536, 6.5 / 2688, 93)}[case]
        x = synth.bf16_normal((rows, k), 1.5, seed, synth.S_X)
        x[1] = 0                                  # an all-zero row
        x[2, :16] = 0x8000                        # a block of -0
    c, sc = nv.quantize_act(bf16_dev(x), _scale_dev(s))
    torch.cuda.synchronize()
    oc, osc = ONV.quantize_act(x, np.float32(s))
    assert np.array_equal(c.cpu().numpy(), oc)
    assert np.array_equal(sc.cpu().numpy(), osc)


def _calibrated_scales(x, ids, gate, up, k):
    """Synthetic calibration as the model card describes its policy: per expert the
    amax of the projection's input over the rows routed to it, the 99th percentile
    across experts, a 5% margin, divided by 6 * 448. Computed with the oracle's
    BF16 path (an input recipe for both sides)."""
    E = gate[0].shape[0]
    ax, ah = [], []
    for e in range(E):
        t = np.nonzero((ids == e).any(axis=1))[0]
        if t.size == 0:
            continue
        xe = x[t]
        ax.append(np.max(np.abs(F.bf16_to_f32(xe))))
        h = OM.linear_gated(xe, (gate[0][e], gate[1][e], gate[2][e]), (up[0][e], up[1][e], up[2][e]))
        ah.append(np.max(np.abs(h)))
    f = lambda a: np.float32(1.05 * np.percentile(a, 99) / 2688.0)
    return f(ax), f(ah)


@pytest.mark.parametrize("T,k,E,H,I,seed,layout", [
    (8, 4, 16, 2048, 512, 94, 0),      # 32 slots: K-split gate/up on 4-row tiles
    (64, 8, 32, 512, 1536, 95, 1),     # decode tiles, resident-H down (K = 1536), tiled weights
    (300, 4, 6, 512, 256, 96, 0),      # prefill tiles, full and ragged
    (150, 8, 40, 256, 512, 97, 1),     # prefill tiles, ~30 rows per expert, tiled weights
    (16, 4, 16, 4096, 192, 98, 0),     # tensor-parallel shard I/8 = 192: down K=192 on the decode kernel
    (300, 4, 6, 512, 192, 99, 0),      # the same shard on prefill tiles (partial last stage)
])
def test_moe_w4a4_vs_oracle(T, k, E, H, I, seed, layout):
    note(f"moe w4a4 T={T} k={k} E={E} H={H} I={I} layout={layout}")
    x, ids, w, gate, up, down = _moe_problem(T, k, E, H, I, seed, sigma=0.05)
    s_gu, s_d = _calibrated_scales(x, ids, gate, up, k)
    y = nv.moe_grouped(bf16_dev(x), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV),
                       weight_dev(gate, layout), weight_dev(up, layout), weight_dev(down, layout),
                       input_scales=_scale_dev(s_gu, s_d))
    torch.cuda.synchronize()
    ref = OM.moe_w4a4(x, ids, w, gate, up, down, s_gu, s_d)
    assert_close(bf16_host_f64(y), ref, "moe w4a4")
    # the W4A4 result differs from the W4A16 one by the activation quantization,
    # and only by it: W4A16 on the same weights is a different (closer to BF16) answer
    ref16 = OM.moe(x, ids, w, gate, up, down)
    assert np.max(np.abs(ref - ref16)) > 1e-3 * np.max(np.abs(ref16))


# ------------------------------------------------------------------ router, shared expert, MoE block
from oracle import block as OB  # noqa: E402


def _margins(lg, k):
    """Smallest gap among the k + 1 largest logits of each row, relative to the row's max |logit|."""
    s = -np.sort(-lg, axis=1)[:, :k + 1]
    return np.min(s[:, :-1] - s[:, 1:], axis=1) / np.max(np.abs(lg), axis=1)


def _router_case(T, E, H, seed):
    x = synth.bf16_normal((T, H), 1.0, seed, synth.S_X)
    wr = synth.bf16_normal((E, H), 0.02, seed, 77)
    return x, wr


@pytest.mark.parametrize("T,E,H,k,seed", [(5, 16, 256, 4, 100), (64, 288, 4096, 8, 101), (300, 288, 4096, 8, 102)])
def test_router_topk_vs_oracle(T, E, H, k, seed):
    note(f"router T={T} E={E} H={H} k={k}")
    x, wr = _router_case(T, E, H, seed)
    ids, w = nv.router_topk(bf16_dev(x), bf16_dev(wr), k)
    torch.cuda.synchronize()
    ids, w = ids.cpu().numpy(), w.cpu().numpy().astype(np.float64)
    oid, ow, lg = OB.router(x, wr, k)
    # where the oracle's top k + 1 logits are separated by more than the fp32 sum's
    # error (~1e-5 of the row scale here), the choice and order are unique
    clear = _margins(lg, k) > 1e-4
    assert clear.mean() > 0.9
    assert np.array_equal(ids[clear], oid[clear])
    assert np.allclose(w[clear], ow[clear], rtol=2e-5, atol=1e-6)
    # elsewhere: k distinct experts whose logits are within the error of the oracle's top
    # k, listed in decreasing logit order (up to that error), with the softmax of their
    # logits as weights
    for t in np.nonzero(~clear)[0]:
        tol = 1e-4 * np.max(np.abs(lg[t]))
        assert len(set(ids[t].tolist())) == k
        kth = np.sort(lg[t])[-k]
        chosen = lg[t, ids[t]]
        assert np.all(chosen >= kth - tol)
        assert np.all(chosen[:-1] >= chosen[1:] - tol), f"row {t}: ids not in decreasing logit order"
        sm = np.exp(chosen - chosen.max())
        assert np.allclose(w[t], sm / sm.sum(), rtol=1e-3, atol=1e-6), f"row {t}: weights not the softmax"


@pytest.mark.parametrize("M,H,Is,seed", [(1, 4096, 1536, 103), (64, 4096, 1536, 104), (300, 2048, 512, 105),
                                         (1024, 1024, 2048, 106),
                                         (4096, 2048, 2048, 109),    # both products on 128-row tiles
                                         # no K split, two-set register ring with odd stage counts: the gated
                                         # product on 64-row tiles (19 stages), down on 128-row tiles (13)
                                         (4096, 1216, 832, 121)])
def test_bf16_mlp_vs_oracle(M, H, Is, seed):
    note(f"bf16 mlp M={M} H={H} Is={Is}")
    x = synth.bf16_normal((M, H), 1.0, seed, synth.S_X)
    sg, su, sd = (synth.bf16_normal(s, 0.02, seed, 80 + i) for i, s in enumerate([(Is, H), (Is, H), (H, Is)]))
    y = nv.bf16_mlp(bf16_dev(x), bf16_dev(sg), bf16_dev(su), bf16_dev(sd))
    torch.cuda.synchronize()
    assert_close(y.cpu().numpy(), OB.shared_mlp(x, sg, su, sd), "bf16 mlp")


@pytest.mark.parametrize("T,k,E,H,I,Is,seed", [(8, 4, 16, 2048, 512, 512, 107), (300, 4, 16, 512, 256, 256, 108)])
def test_moe_block_vs_oracle(T, k, E, H, I, Is, seed):
    note(f"moe block T={T} k={k} E={E} H={H} I={I} Is={Is}")
    x, wr = _router_case(T, E, H, seed)
    gate = ONV.pack_batch(synth.expert_weights(E, I, H, 0.05, seed, synth.S_GATE))
    up = ONV.pack_batch(synth.expert_weights(E, I, H, 0.05, seed, synth.S_UP))
    down = ONV.pack_batch(synth.expert_weights(E, H, I, 0.05, seed, synth.S_DOWN))
    sg, su, sd = (synth.bf16_normal(s, 0.05, seed, 90 + i) for i, s in enumerate([(Is, H), (Is, H), (H, Is)]))
    y_ref, oid, _, lg = OB.moe_block(x, wr, k, gate, up, down, sg, su, sd)
    assert _margins(lg, k).min() > 1e-4          # the routing is unique for this input
    y = nv.moe_block(bf16_dev(x), bf16_dev(wr), k, weight_dev(gate), weight_dev(up), weight_dev(down),
                     bf16_dev(sg), bf16_dev(su), bf16_dev(sd))
    torch.cuda.synchronize()
    assert_close(bf16_host_f64(y), y_ref, "moe block")


# ------------------------------------------------------------------ edge cases of the added entry points
def test_moe_w4a4_expert_parallel_slice_duplicates_and_saturation():
    # expert_begin 4 of 12 ids, duplicate ids, and an input scale small enough that
    # most blocks of x saturate (byte 0x7E, codes clamped at 6)
    T, k, E, H, I = 30, 4, 4, 256, 256
    g = np.random.default_rng(5)
    ids = g.integers(0, 12, (T, k)).astype(np.int32)
    ids[:, 1] = ids[:, 0]
    w = g.uniform(0.1, 1.0, (T, k)).astype(np.float32)
    x, _, _, gate, up, down = _moe_problem(T, k, E, H, I, 109, sigma=0.05, ids=ids, weights=w)
    s_gu, s_d = np.float32(0.5 / 2688), np.float32(4.0 / 2688)
    y = nv.moe_grouped(bf16_dev(x), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV), weight_dev(gate),
                       weight_dev(up), weight_dev(down), expert_begin=4, input_scales=_scale_dev(s_gu, s_d))
    torch.cuda.synchronize()
    ref = OM.moe_w4a4(x, ids, w, gate, up, down, s_gu, s_d, expert_begin=4)
    assert_close(bf16_host_f64(y), ref, "moe w4a4 ep slice")
    _, sc = ONV.quantize_act(x, s_gu)
    assert (sc == 0x7E).mean() > 0.5          # the saturating case is exercised


def test_moe_w4a4_token_permutation_and_repeat_bitwise():
    T, k, E, H, I = 64, 8, 32, 512, 1536
    x, ids, w, gate, up, down = _moe_problem(T, k, E, H, I, 110, sigma=0.05)
    sc = _scale_dev(4.0 / 2688, 1.0 / 2688)
    run = lambda xx, ii, ww: bf16_host_bits(nv.moe_grouped(
        bf16_dev(xx), torch.from_numpy(ii).to(DEV), torch.from_numpy(ww).to(DEV), weight_dev(gate, 1),
        weight_dev(up, 1), weight_dev(down, 1), input_scales=sc))
    y1, y2 = run(x, ids, w), run(x, ids, w)
    assert np.array_equal(y1, y2)
    p = np.random.default_rng(2).permutation(T)
    assert np.array_equal(run(x[p], ids[p], w[p]), y1[p])


def test_moe_w4a4_rejects_fallback_shapes():
    # H = 128 is covered only by the fallback GEMM, which has no W4A4 form
    x, ids, w, gate, up, down = _moe_problem(8, 2, 4, 128, 64, 111)
    with pytest.raises(RuntimeError):
        nv.moe_grouped(bf16_dev(x), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV), weight_dev(gate),
                       weight_dev(up), weight_dev(down), input_scales=_scale_dev(0.01, 0.01))


@pytest.mark.parametrize("T,E,k", [(1, 20, 20), (3, 20, 1), (33, 8, 2)])
def test_router_small_and_all_experts(T, E, k):
    note(f"router T={T} E={E} k={k}")
    x, wr = _router_case(T, E, 256, 112 + E + k)
    ids, w = nv.router_topk(bf16_dev(x), bf16_dev(wr), k)
    torch.cuda.synchronize()
    oid, ow, lg = OB.router(x, wr, k)
    assert _margins(lg, min(k, E - 1)).min() > 1e-4
    assert np.array_equal(ids.cpu().numpy(), oid)
    assert np.allclose(w.cpu().numpy(), ow, rtol=2e-5, atol=1e-6)


@pytest.mark.parametrize("T,k,E,H,I,Is,seed", [(1, 4, 16, 512, 256, 256, 113),    # K-split gate/up, decode down
                                                (2, 4, 16, 512, 512, 256, 114)])   # the two-launch path
def test_moe_block_single_token(T, k, E, H, I, Is, seed):
    x, wr = _router_case(T, E, H, seed)
    gate = ONV.pack_batch(synth.expert_weights(E, I, H, 0.05, seed, synth.S_GATE))
    up = ONV.pack_batch(synth.expert_weights(E, I, H, 0.05, seed, synth.S_UP))
    down = ONV.pack_batch(synth.expert_weights(E, H, I, 0.05, seed, synth.S_DOWN))
    sg, su, sd = (synth.bf16_normal(s, 0.05, seed, 90 + i) for i, s in enumerate([(Is, H), (Is, H), (H, Is)]))
    y_ref, _, _, lg = OB.moe_block(x, wr, k, gate, up, down, sg, su, sd)
    assert _margins(lg, k).min() > 1e-4
    y = nv.moe_block(bf16_dev(x), bf16_dev(wr), k, weight_dev(gate), weight_dev(up), weight_dev(down),
                     bf16_dev(sg), bf16_dev(su), bf16_dev(sd))
    torch.cuda.synchronize()
    assert_close(bf16_host_f64(y), y_ref, f"moe block T={T}")


# ------------------------------------------------------------------ BF16 routed experts
@pytest.mark.parametrize("T,k,E,H,I,seed,eb", [
    (8, 4, 16, 2048, 512, 114, 0),      # decode-like: ~2 rows per expert
    (300, 4, 6, 512, 256, 115, 0),      # 200 rows per expert: 128-row tiles, the second ragged
    (600, 8, 5, 256, 128, 118, 0),      # 4800 slots: windowed route, 128-row tiles
    (40, 4, 16, 256, 128, 119, 0),      # 10 rows per expert: 64-row tiles
    (1, 8, 12, 256, 128, 116, 0),       # one token
    (30, 4, 4, 256, 128, 117, 4),       # expert-parallel slice (ids 0..11, local 4..7), duplicates
    (300, 4, 6, 1216, 832, 120, 0),     # 128-row tiles with K loops of 19 and 13 stages (two-set register ring)
])
def test_moe_grouped_bf16_vs_oracle(T, k, E, H, I, seed, eb):
    note(f"moe bf16 T={T} k={k} E={E} H={H} I={I} eb={eb}")
    x = synth.bf16_normal((T, H), 1.0, seed, synth.S_X)
    if eb:
        g = np.random.default_rng(seed)
        ids = g.integers(0, 3 * E, (T, k)).astype(np.int32)
        ids[:, 1] = ids[:, 0]
        w = g.uniform(0.1, 1.0, (T, k)).astype(np.float32)
    else:
        ids, w = synth.topk_softmax_routing(T, E, k, seed, synth.S_ROUTE)
    wg = synth.expert_weights(E, I, H, 0.05, seed, synth.S_GATE)
    wu = synth.expert_weights(E, I, H, 0.05, seed, synth.S_UP)
    wd = synth.expert_weights(E, H, I, 0.05, seed, synth.S_DOWN)
    y = nv.moe_grouped_bf16(bf16_dev(x), torch.from_numpy(ids.astype(np.int32)).to(DEV),
                            torch.from_numpy(w.astype(np.float32)).to(DEV), bf16_dev(wg), bf16_dev(wu), bf16_dev(wd),
                            expert_begin=eb)
    torch.cuda.synchronize()
    ref = OB.moe_bf16(x, ids, w, wg, wu, wd, expert_begin=eb)
    assert_close(bf16_host_f64(y), ref, "moe bf16")
