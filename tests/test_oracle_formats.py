"""Pins for oracle.formats: bf16, e2m1 and e4m3 against torch's casts, the OCP
value tables and brute-force nearest-value search."""
import numpy as np
import pytest
import torch

from oracle import formats as F


def _torch_bf16_bits(x32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _edge_f32():
    g = np.random.default_rng(11)
    vals = [0.0, -0.0, 1.0, -1.0, 3.4e38, -3.4e38, np.inf, -np.inf, 1e-45, -1e-45, 1.17549435e-38]
    # exact ties of the bf16 rounding: 1 + 2^-8 (tie, even down), 1 + 3*2^-8 (tie, even up)
    vals += [1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -130 * (1 + 2 ** -8)]
    rnd = g.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** g.integers(-30, 30, 20000).astype(np.float32)
    bits = g.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    bits = bits[np.isfinite(bits)]
    return np.concatenate([np.array(vals, np.float32), rnd.astype(np.float32), bits])


def test_bf16_narrow_matches_torch():
    x = _edge_f32()
    assert np.array_equal(F.f32_to_bf16(x), _torch_bf16_bits(x))


def test_bf16_narrow_nan_stays_nan():
    x = np.array([np.nan, -np.nan], np.float32)
    assert np.all(np.isnan(F.bf16_to_f32(F.f32_to_bf16(x))))


def test_bf16_widen_all_patterns_match_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = F.bf16_to_f32(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_generic_minifloat_matches_torch_e4m3fn_all_bytes():
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    ours = F.e4m3_decode(b)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan) and nan.sum() == 2
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_generic_minifloat_matches_torch_e5m2_all_bytes():
    # the same closed form with e5m2 parameters and IEEE specials; pins the formula itself
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e5m2).to(torch.float32).numpy().astype(np.float64)
    ours = F.minifloat_decode(b, 5, 2, 15, "ieee")
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_e2m1_value_table():
    # OCP MX FP4 (E2M1): magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; bit 3 is the sign
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    v = F.e2m1_decode(np.arange(16))
    assert list(v[:8]) == mags
    assert list(-v[8:]) == mags
    assert np.all(np.signbit(v[8:]))


def test_e4m3_special_values():
    assert F.e4m3_decode(0x7E) == 448.0
    assert F.e4m3_decode(0x08) == 2.0 ** -6
    assert F.e4m3_decode(0x01) == 2.0 ** -9
    assert F.e4m3_decode(0x38) == 1.0
    assert np.isnan(F.e4m3_decode(0x7F)) and np.isnan(F.e4m3_decode(0xFF))


def _e4m3_probe_values():
    grid = np.sort(np.unique(F.e4m3_decode(np.arange(0x7F))))          # 0 .. 448
    mids = (grid[:-1] + grid[1:]) / 2
    m32 = mids.astype(np.float32)
    around = np.concatenate([m32, np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(1e9))])
    g = np.random.default_rng(5)
    lin = g.uniform(0, 448, 200000).astype(np.float32)
    log = np.exp2(g.uniform(-14, np.log2(448), 200000)).astype(np.float32)
    v = np.concatenate([grid.astype(np.float32), around, lin, log, np.array([448.0], np.float32)])
    return v[(v >= 0) & (v <= 448)]


def test_e4m3_encode_matches_torch_cast():
    v = _e4m3_probe_values()
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(F.e4m3_encode(v), ref)


def test_e4m3_encode_roundtrip_and_saturation():
    b = np.arange(0x7F, dtype=np.uint8)
    assert np.array_equal(F.e4m3_encode(F.e4m3_decode(b).astype(np.float32)), b)
    big = np.array([448.0, 449.0, 464.0, 480.0, 1e6, 3e38], np.float32)
    assert np.all(F.e4m3_encode(big) == 0x7E)
    # underflow: at or below half the smallest subnormal goes to zero (tie to even)
    assert F.e4m3_encode(np.float32(2.0 ** -10)) == 0
    assert F.e4m3_encode(np.float32(np.nextafter(np.float32(2.0 ** -10), np.float32(1)))) == 1


def _nearest_e2m1(q: float) -> int:
    """Brute force: nearest representable magnitude (<= 6), ties to the even index."""
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    a = min(abs(float(q)), 6.0)
    d = [abs(a - m) for m in mags]
    best = min(d)
    cands = [i for i in range(8) if d[i] == best]
    idx = cands[0] if len(cands) == 1 else [i for i in cands if i % 2 == 0][0]
    return idx | (8 if np.signbit(q) else 0)


def test_e2m1_encode_vs_nearest_search():
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    around = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(10))])
    g = np.random.default_rng(3)
    vals = np.concatenate([around, -around, g.uniform(-8, 8, 5000).astype(np.float32),
                           np.array([0.0, -0.0, 6.0, -6.0, 6.4, -6.4, 100.0, 1e-30, -1e-30], np.float32),
                           F.e2m1_decode(np.arange(16)).astype(np.float32)])
    ours = F.e2m1_encode(vals)
    ref = np.array([_nearest_e2m1(v) for v in vals], np.uint8)
    assert np.array_equal(ours, ref)


@pytest.mark.parametrize("q,code", [(0.25, 0x0), (0.75, 0x2), (1.25, 0x2), (1.75, 0x4), (2.5, 0x4),
                                    (3.5, 0x6), (5.0, 0x6), (-0.0, 0x8), (-0.2, 0x8), (6.5, 0x7), (-7.0, 0xF)])
def test_e2m1_encode_ties_and_signs(q, code):
    assert F.e2m1_encode(np.float32(q)) == code


def test_e2m1_encode_decode_roundtrip():
    c = np.arange(16, dtype=np.uint8)
    assert np.array_equal(F.e2m1_encode(F.e2m1_decode(c).astype(np.float32)), c)
