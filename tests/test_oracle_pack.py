"""Pins for oracle.nvfp4: hand-derived golden bytes, invariants of the recipe,
the round-trip bound, degenerate tensors, and exhaustive dequant exactness."""
import json
import os

import numpy as np
import pytest

import synth
from oracle import brute, formats as F, nvfp4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pack_small.json")


def _golden():
    with open(GOLDEN) as f:
        g = json.load(f)
    w = np.zeros(g["w_bf16"]["shape"], np.uint16)
    for r, c, h in g["w_bf16"]["nonzero"]:
        w[r, c] = int(h, 16)
    codes = np.array([[int(h, 16) for h in row] for row in g["codes"]], np.uint8)
    scales = np.array([[int(h, 16) for h in row] for row in g["scales"]], np.uint8)
    s2 = np.uint32(int(g["scale_2_bits"], 16)).view(np.float32)
    return w, codes, scales, s2


def test_pack_golden_hand_derived():
    w, codes, scales, s2 = _golden()
    c, s, x = nvfp4.pack(w)
    assert np.array_equal(c, codes)
    assert np.array_equal(s, scales)
    assert np.float32(x).view(np.uint32) == s2.view(np.uint32)


def _tensors():
    out = []
    for i, (n, k, sigma) in enumerate([(64, 256, 0.02), (33, 512, 1.0), (8, 4096, 0.02), (128, 64, 3e-3),
                                       (16, 1536, 0.02), (7, 32, 100.0)]):
        out.append(synth.bf16_normal((n, k), sigma, 900, i))
    # heavy-tailed and mixed-magnitude rows
    g = np.random.default_rng(4)
    z = (g.standard_cauchy((24, 256)) * 0.01).astype(np.float32)
    out.append(synth.f32_to_bf16_bits(z))
    z = (g.standard_normal((24, 256)) * np.exp2(g.integers(-20, 6, (24, 1)))).astype(np.float32)
    out.append(synth.f32_to_bf16_bits(z))
    return out


@pytest.mark.parametrize("ti", range(8))
def test_pack_invariants(ti):
    w = _tensors()[ti]
    codes, scales, s2 = nvfp4.pack(w)
    wf = F.bf16_to_f32(w)
    N, K = w.shape
    # (iii) no scale byte above 0x7E (no NaN, no negative)
    assert scales.max() <= 0x7E
    # (i) the block holding amax gets the saturated byte (v ~ 448)
    assert scales.max() == 0x7E
    blocks = np.abs(wf).reshape(N, K // 16, 16)
    bamax = blocks.max(axis=2)
    r, b = np.unravel_index(np.argmax(bamax), bamax.shape)
    assert scales[r, b] == 0x7E
    # (ii) blocks with a normal scale byte have |code| == 6 at their largest element
    codes4 = nvfp4.unpack_codes(codes).reshape(N, K // 16, 16)
    arg = blocks.argmax(axis=2)
    top = np.take_along_axis(codes4, arg[..., None], axis=2)[..., 0] & 7
    normal = scales >= 0x08
    assert np.all(top[normal] == 7)
    # (iv) round-trip bound per element
    u, wq = nvfp4.dequant(codes, scales, s2)
    s_eff = (F.e4m3_decode(scales).astype(np.float32) * s2).astype(np.float64)
    s_eff = np.repeat(s_eff, 16, axis=1)
    mag = np.abs(F.e2m1_decode(nvfp4.unpack_codes(codes)))
    gap = np.select([mag < 2, mag < 4, mag < 6], [0.5, 1.0, 2.0], 2.0)
    q = np.abs(wf.astype(np.float64)) / np.where(s_eff > 0, s_eff, 1)
    bound = np.where(q > 6, (q - 6) * s_eff, 0.5 * gap * s_eff) + 4e-7 * np.abs(wf) + 1e-45
    live = s_eff > 0
    assert np.all((np.abs(wf - wq.astype(np.float64)) <= bound)[live])
    # a block whose scale byte rounded to 0 had v <= 2^-10, i.e. |w| <= 6 * 2^-10 * scale_2,
    # and dequantizes to exactly 0
    assert np.all(wq[~live] == 0)
    assert np.all(np.abs(wf[~live]) <= 6 * 2.0 ** -10 * float(s2) * (1 + 1e-6))


def test_pack_scale_bytes_vs_float64_rederivation():
    # recompute v in float64; a different byte is allowed only where the fp32
    # value sits within a few ulps of an e4m3 rounding midpoint
    for w in _tensors():
        _, scales, s2 = nvfp4.pack(w)
        wf = F.bf16_to_f32(w).astype(np.float64)
        N, K = w.shape
        bamax = np.abs(wf).reshape(N, K // 16, 16).max(axis=2)
        v64 = bamax / 6.0 / float(s2)
        b64 = F.e4m3_encode(np.minimum(v64, 448.0).astype(np.float32))
        diff = b64 != scales
        if np.any(diff):
            lo = F.e4m3_decode(np.minimum(scales[diff], b64[diff]))
            hi = F.e4m3_decode(np.maximum(scales[diff], b64[diff]))
            mid = (lo + hi) / 2
            assert np.all(np.abs(v64[diff] - mid) <= 8 * np.spacing(np.float32(mid)).astype(np.float64))


def test_pack_zero_tensor_and_zero_blocks():
    z = np.zeros((4, 64), np.uint16)
    c, s, s2 = nvfp4.pack(z)
    assert s2 == 0 and not c.any() and not s.any()
    w = synth.bf16_normal((4, 64), 0.02, 901)
    w[:, 16:32] = 0                       # one all-zero block per row
    w[2, :] = 0x8000                      # a row of negative zeros
    c, s, s2 = nvfp4.pack(w)
    assert s2 > 0
    assert not s[:, 1].any() and not c[:, 8:16].any()
    assert not s[2].any() and not c[2].any()


def test_pack_negative_zero_inside_nonzero_block():
    w = np.zeros((1, 32), np.uint16)
    w[0, 0] = 0x3F80     # 1.0
    w[0, 1] = 0x8000     # -0.0 -> q = -0.0 -> sign bit set -> code 0x8
    c, s, _ = nvfp4.pack(w)
    assert c[0, 0] == (0x7 | (0x8 << 4))


def test_pack_tiny_and_subnormal_magnitudes():
    # bf16 subnormals and a tensor whose scale bytes land in the e4m3 subnormal range
    w = np.zeros((2, 32), np.uint16)
    w[0, 0] = 0x0001                      # smallest bf16 subnormal
    w[1, 0] = 0x3F80                      # 1.0 makes scale_2 ~ 1/2688
    w[1, 16] = 0x3780                     # 2^-16: v = 2^-16*448 ~ 0.0068 < 2^-6 -> subnormal e4m3 byte
    c, s, s2 = nvfp4.pack(w)
    assert s2 > 0 and s[1, 0] == 0x7E and 0 < s[1, 1] < 0x08
    c1, s1, t2 = nvfp4.pack(w[:1])
    assert t2 > 0 and s1[0, 0] == 0x7E and (c1[0, 0] & 7) == 7


def test_pack_batch_independent_scale2():
    ws = np.stack([synth.bf16_normal((16, 64), s, 902, i) for i, s in enumerate([0.02, 1.0, 5e-4])])
    c, s, s2 = nvfp4.pack_batch(ws)
    for g in range(3):
        c1, sg, s21 = nvfp4.pack(ws[g])
        assert np.array_equal(c[g], c1) and np.array_equal(s[g], sg) and s2[g] == s21
    assert len(set(s2.tolist())) == 3


def test_dequant_exhaustive_pairs_exact():
    # all 16 x 256 (code, scale byte) pairs; finite scale bytes only
    codes = np.arange(16, dtype=np.uint8)
    sb = np.array([b for b in range(256) if b not in (0x7F, 0xFF)], np.uint8)
    cc = np.repeat(codes, 16)                       # 16 copies so one scale byte covers a block
    packed = (cc[0::2] | (cc[1::2] << 4)).astype(np.uint8)        # [128] bytes = 256 codes
    for b in sb:
        scales = np.full((1, 256 // 16), b, np.uint8)
        u, wq = nvfp4.dequant(packed[None, :], scales, np.float32(1.0))
        ref = np.array([brute._e2m1(int(c)) * brute._e4m3(int(b)) for c in cc])
        assert np.array_equal(u[0].astype(np.float64), ref)
        # the unscaled product is exact in bf16
        assert np.array_equal(F.bf16_to_f32(F.f32_to_bf16(u[0])), u[0])


def test_dequant_scaled_single_rounding():
    w = synth.bf16_normal((8, 128), 0.02, 903)
    c, s, s2 = nvfp4.pack(w)
    u, wq = nvfp4.dequant(c, s, s2)
    assert np.array_equal(wq, (u.astype(np.float64) * float(s2)).astype(np.float32))


def test_nibble_order_against_brute_weight():
    w = synth.bf16_normal((5, 64), 0.02, 904)
    c, s, s2 = nvfp4.pack(w)
    _, wq = nvfp4.dequant(c, s, s2)
    for n in range(5):
        for k in range(64):
            assert np.float32(brute.weight(c, s, s2, n, k)) == wq[n, k]
