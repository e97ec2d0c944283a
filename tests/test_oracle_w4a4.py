"""Pins for the W4A4 additions of the oracle: static activation quantization
(oracle.nvfp4.quantize_act) and the routed MLP with quantized activations
(oracle.mlp.moe_w4a4).

quantize_act is pinned by: agreement with the pack when the input scale is the
pack's own scale_2; an exact round trip of activations built on the NVFP4 grid
from the format closed forms; hand-derived saturation bytes; and the rounding
bound of every element. moe_w4a4 is pinned by its reduction, for k = 1 and
on-grid inputs, to the already pinned dense pieces (oracle.mlp.linear, silu),
and by its invariants."""
import numpy as np
import pytest

import synth
from oracle import formats as F, mlp, nvfp4

E2M1 = F.e2m1_decode(np.arange(16))
E4M3 = F.e4m3_decode(np.arange(256))


def _on_grid(M, K, in_scale_pow2, seed):
    """bf16 activations whose static quantization is known without the recipe:
    every block holds one code of magnitude 6 (so its amax is 6 * e4m3(b) * s and
    the block's scale byte is b exactly), the other codes are random; s is a power
    of two so every value (<= 6 significant bits) is exact in bf16."""
    g = np.random.default_rng(seed)
    nb = K // 16
    byte = g.integers(0x10, 0x70, (M, nb)).astype(np.uint8)       # normal e4m3 bytes
    code = g.integers(0, 16, (M, K)).astype(np.uint8)
    pos = g.integers(0, 16, (M, nb))
    for m in range(M):
        for b in range(nb):
            code[m, 16 * b + pos[m, b]] = 0x7 | (code[m, 16 * b + pos[m, b]] & 0x8)   # +-6
    vals = E2M1[code] * np.repeat(E4M3[byte], 16, axis=1) * in_scale_pow2
    bits = F.f32_to_bf16(vals.astype(np.float32))
    assert np.array_equal(F.bf16_to_f32(bits).astype(np.float64), vals)   # exact
    return bits, code, byte


def test_quantize_act_equals_pack_at_the_pack_scale():
    w = synth.bf16_normal((24, 128), 0.7, 950)
    c, s, s2 = nvfp4.pack(w)
    ca, sa = nvfp4.quantize_act(w, s2)
    assert np.array_equal(ca, c) and np.array_equal(sa, s)


@pytest.mark.parametrize("s", [1.0, 2.0 ** -6, 2.0 ** 3])
def test_quantize_act_round_trip_on_grid(s):
    bits, code, byte = _on_grid(7, 256, s, 951)
    codes, scales = nvfp4.quantize_act(bits, np.float32(s))
    assert np.array_equal(scales, byte)
    got = nvfp4.unpack_codes(codes)
    # -0 encodes with its sign bit; compare values, and codes where nonzero
    nz = (code & 7) != 0
    assert np.array_equal(got[nz], code[nz])
    assert np.all((got[~nz] & 7) == 0)


def test_quantize_act_saturation_hand_derived():
    # input_scale 1/64: the largest representable magnitude is 6 * 448 / 64 = 42.
    # A block of 100.0 needs v = 100/6*64 = 1066.7 > 448: byte 0x7E, every code +6
    # (0x7). A block of -0.5 has v = 0.5/6*64 = 5.333.., whose e4m3 neighbours are
    # 5.0 (0x4A) and 5.5 (0x4B): nearest is 5.5 (0x4B); s_eff = 5.5/64, q = -0.5 /
    # (5.5/64) = -5.8181.. -> code 6 with the sign: 0xF.
    x = np.zeros((1, 48), np.float32)
    x[0, :16] = 100.0
    x[0, 16:32] = -0.5
    bits = F.f32_to_bf16(x)
    codes, scales = nvfp4.quantize_act(bits, np.float32(1.0 / 64))
    assert list(scales[0]) == [0x7E, 0x4B, 0x00]
    c = nvfp4.unpack_codes(codes)[0]
    assert np.all(c[:16] == 0x7) and np.all(c[16:32] == 0xF) and np.all(c[32:] == 0)


def test_quantize_act_zero_scale_and_zero_rows():
    x = synth.bf16_normal((3, 64), 1.0, 952)
    codes, scales = nvfp4.quantize_act(x, np.float32(0.0))
    assert not codes.any() and not scales.any()
    codes, scales = nvfp4.quantize_act(np.zeros((2, 32), np.uint16), np.float32(0.01))
    assert not codes.any() and not scales.any()


def test_quantize_act_rounding_bound():
    # every element lies within half a local e2m1 gap of its quantized value (or is
    # clamped at 6), measured in units of the block's effective scale
    x = synth.bf16_normal((16, 256), 2.0, 953)
    s = np.float32(3.0 / 2688)                     # some blocks saturate, most do not
    codes, scales = nvfp4.quantize_act(x, s)
    xv = F.bf16_to_f32(x).astype(np.float64)
    s_eff = (E4M3[scales].astype(np.float32) * s).astype(np.float64)
    q = xv / np.repeat(s_eff, 16, axis=1)
    got = E2M1[nvfp4.unpack_codes(codes)]
    mag = np.abs(q)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    gap = np.array([0.5, 0.5, 0.5, 0.5, 1, 1, 2, 2])
    idx = np.clip(np.searchsorted(grid, np.minimum(mag, 6.0), side="right") - 1, 0, 7)
    bound = 0.5 * gap[idx] + 1e-6 * np.maximum(mag, 1)
    ok = (np.abs(np.abs(got) - mag) <= bound) | ((mag >= 6) & (np.abs(got) == 6))
    assert ok.all()
    assert np.all(np.sign(got)[mag > 0.25] == np.sign(q)[mag > 0.25])


def _tiny_moe(T, k, E, H, I, seed, sigma=0.3):
    ids, w = synth.topk_softmax_routing(T, E, k, seed, 1)
    gate = nvfp4.pack_batch(synth.bf16_normal((E, I, H), sigma, seed, 2))
    up = nvfp4.pack_batch(synth.bf16_normal((E, I, H), sigma, seed, 3))
    down = nvfp4.pack_batch(synth.bf16_normal((E, H, I), sigma, seed, 4))
    return ids, w, gate, up, down


def test_moe_w4a4_k1_reduces_to_pinned_dense_pieces():
    # k = 1, weight 1, x on the grid of its input scale (so its quantization is the
    # identity): y_t = s_d * linear(e2m1 * e4m3 of quantize(bf16(silu(g) * u)), Wd)
    # with g, u from the pinned linear
    T, E, H, I = 6, 3, 64, 32
    s_gu, s_d = np.float32(2.0 ** -4), np.float32(0.37 / 2688)
    ids, _, gate, up, down = _tiny_moe(T, 1, E, H, I, 954)
    w = np.ones((T, 1), np.float32)
    x, _, _ = _on_grid(T, H, float(s_gu), 955)
    y = mlp.moe_w4a4(x, ids, w, gate, up, down, s_gu, s_d)
    for t in range(T):
        e = int(ids[t, 0])
        ex = lambda p: (p[0][e], p[1][e], p[2][e])
        g = mlp.linear(x[t:t + 1], ex(gate))
        u = mlp.linear(x[t:t + 1], ex(up))
        hb = F.f32_to_bf16((mlp.silu(g) * u).astype(np.float32))
        c, sc = nvfp4.quantize_act(hb, s_d)
        hu = nvfp4.dequant_unscaled(c, sc)          # e2m1 * e4m3: 6 bits, exact in bf16
        hu_bits = F.f32_to_bf16(hu.astype(np.float32))
        assert np.array_equal(F.bf16_to_f32(hu_bits).astype(np.float64), hu)
        yt = np.float64(s_d) * mlp.linear(hu_bits, ex(down))
        assert np.allclose(y[t], yt[0], rtol=1e-12, atol=1e-15)


def test_moe_w4a4_invariants():
    T, k, E, H, I = 9, 2, 4, 32, 32
    ids, w, gate, up, down = _tiny_moe(T, k, E, H, I, 956)
    x = synth.bf16_normal((T, H), 1.0, 957)
    s_gu, s_d = np.float32(4.0 / 2688), np.float32(0.5 / 2688)
    y = mlp.moe_w4a4(x, ids, w, gate, up, down, s_gu, s_d)
    # token permutation permutes the output exactly
    p = np.random.default_rng(958).permutation(T)
    yp = mlp.moe_w4a4(x[p], ids[p], w[p], gate, up, down, s_gu, s_d)
    assert np.array_equal(yp, y[p])
    # zero routing weights give exactly zero
    assert not mlp.moe_w4a4(x, ids, np.zeros_like(w), gate, up, down, s_gu, s_d).any()
    # skipped ids contribute nothing
    y_skip = mlp.moe_w4a4(x, ids, w, gate, up, down, s_gu, s_d, expert_begin=E)
    assert not y_skip.any()
