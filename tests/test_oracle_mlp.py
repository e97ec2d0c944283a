"""Pins for oracle.mlp: brute force, exact integer arithmetic, library sorts,
and the algebraic properties of the routed MLP."""
import numpy as np
import pytest

import synth
from oracle import brute, formats as F, mlp, nvfp4


def _packed(n, k, sigma, *key):
    return nvfp4.pack(synth.bf16_normal((n, k), sigma, *key))


@pytest.mark.parametrize("M,N,K", [(2, 3, 32), (3, 5, 64), (1, 4, 48)])
def test_linear_vs_brute(M, N, K):
    x = synth.bf16_normal((M, K), 1.0, 910, M, N, K)
    c, s, s2 = _packed(N, K, 0.02, 911, M, N, K)
    y = mlp.linear(x, (c, s, s2))
    yb = np.array(brute.linear(x.tolist(), c.tolist(), s.tolist(), s2, M, N, K))
    assert y.shape == (M, N)
    assert np.allclose(y, yb, rtol=1e-12, atol=1e-14)


def test_linear_integer_exact():
    # scale bytes 1.0, scale_2 1.0, x integers in [-8, 8]: every product and sum is
    # an exact multiple of 0.5, so the result must equal integer arithmetic exactly
    g = np.random.default_rng(12)
    M, N, K = 4, 6, 512
    x = synth.bf16_integers((M, K), -8, 8, 913)
    codes4 = g.integers(0, 16, (N, K)).astype(np.uint8)
    codes = (codes4[:, 0::2] | (codes4[:, 1::2] << 4)).astype(np.uint8)
    scales = np.full((N, K // 16), 0x38, np.uint8)
    y = mlp.linear(x, (codes, scales, np.float32(1.0)))
    twice = {0: 0, 1: 1, 2: 2, 3: 3, 4: 4, 5: 6, 6: 8, 7: 12}          # 2 * e2m1 magnitude
    w2 = np.array([[(-1 if c & 8 else 1) * twice[c & 7] for c in row] for row in codes4], np.int64)
    xi = F.bf16_to_f32(x).astype(np.int64)
    exact2 = xi @ w2.T
    assert np.array_equal(y * 2, exact2.astype(np.float64))


def test_linear_gated_vs_brute():
    M, I, H = 2, 3, 32
    x = synth.bf16_normal((M, H), 1.0, 914)
    wg = _packed(I, H, 0.5, 915)
    wu = _packed(I, H, 0.5, 916)
    h = mlp.linear_gated(x, wg, wu)
    g = brute.linear(x.tolist(), wg[0].tolist(), wg[1].tolist(), wg[2], M, I, H)
    u = brute.linear(x.tolist(), wu[0].tolist(), wu[1].tolist(), wu[2], M, I, H)
    hb = np.array([[brute.silu(g[m][i]) * u[m][i] for i in range(I)] for m in range(M)])
    assert np.allclose(h, hb, rtol=1e-12, atol=1e-15)


def test_silu_closed_form_values():
    z = np.array([0.0, 1.0, -1.0, 20.0, -800.0])
    ref = np.array([0.0, 1 / (1 + np.exp(-1.0)), -1 / (1 + np.exp(1.0)), 20 / (1 + np.exp(-20.0)), 0.0])
    assert np.allclose(mlp.silu(z), ref, rtol=1e-15, atol=0)


def _brute_route(ids, E, eb):
    flat = [int(v) for v in np.asarray(ids).reshape(-1)]
    perm = []
    for e in range(E):
        perm += [s for s, v in enumerate(flat) if v - eb == e]
    counts = [sum(1 for v in flat if v - eb == e) for e in range(E)]
    inv = [-1] * len(flat)
    for p, s in enumerate(perm):
        inv[s] = p
    return counts, perm, inv


@pytest.mark.parametrize("T,k,E,eb,lo,hi", [(8, 4, 16, 0, 0, 15), (37, 8, 288, 0, 0, 287), (20, 3, 5, 10, 0, 30),
                                              (1, 8, 288, 0, 0, 287), (0, 8, 16, 0, 0, 15), (50, 2, 4, 0, 0, 3)])
def test_route_vs_stable_argsort_and_brute(T, k, E, eb, lo, hi):
    g = np.random.default_rng(T * 1000 + E)
    ids = g.integers(lo, hi + 1, (T, k)).astype(np.int32)
    counts, offsets, perm, inv = mlp.route(ids, E, eb)
    bc, bp, bi = _brute_route(ids, E, eb)
    assert counts.tolist() == bc and perm.tolist() == bp and inv.tolist() == bi
    flat = ids.reshape(-1).astype(np.int64) - eb
    valid = (flat >= 0) & (flat < E)
    key = np.where(valid, flat, E)                          # skipped slots sort last
    ref = np.argsort(key, kind="stable")[: int(valid.sum())]
    assert np.array_equal(perm, ref)
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts) and offsets[-1] == valid.sum()


def _moe_inputs(T, k, E, H, I, seed, sigma=0.5, ids=None):
    x = synth.bf16_normal((T, H), 1.0, seed, synth.S_X)
    if ids is None:
        ids, w = synth.topk_softmax_routing(T, E, k, seed, synth.S_ROUTE)
    else:
        w = synth.rng(seed, synth.S_RW).uniform(0.1, 1, ids.shape).astype(np.float32)
    gate = nvfp4.pack_batch(synth.expert_weights(E, I, H, sigma, seed, synth.S_GATE))
    up = nvfp4.pack_batch(synth.expert_weights(E, I, H, sigma, seed, synth.S_UP))
    down = nvfp4.pack_batch(synth.expert_weights(E, H, I, sigma, seed, synth.S_DOWN))
    return x, ids, w, gate, up, down


def test_moe_vs_brute():
    T, k, E, H, I = 5, 2, 3, 32, 32
    x, ids, w, gate, up, down = _moe_inputs(T, k, E, H, I, 920)
    ids[0, 1] = ids[0, 0]                                   # duplicate id in a token counts twice
    y = mlp.moe(x, ids, w, gate, up, down)
    yb = np.array(brute.moe(x.tolist(), ids.tolist(), w.tolist(), gate, up, down, T, k, H, I))
    assert np.allclose(y, yb, rtol=1e-10, atol=1e-12)


def test_moe_expert_begin_skips_nonlocal():
    T, k, E, H, I = 4, 3, 3, 32, 32
    ids = np.array([[5, 6, 7], [1, 5, 9], [7, 7, 2], [8, 8, 8]], np.int32)
    x, ids, w, gate, up, down = _moe_inputs(T, k, E, H, I, 921, ids=ids)
    y = mlp.moe(x, ids, w, gate, up, down, expert_begin=5)
    yb = np.array(brute.moe(x.tolist(), ids.tolist(), w.tolist(), gate, up, down, T, k, H, I, expert_begin=5, E=E))
    assert np.allclose(y, yb, rtol=1e-10, atol=1e-12)
    assert np.all(y[3] == 0)


def test_moe_k1_reduces_to_dense_mlp():
    T, E, H, I = 6, 4, 64, 32
    ids = np.array([[2]] * T, np.int32)
    x, ids, _, gate, up, down = _moe_inputs(T, 1, E, H, I, 922, ids=ids)
    w = np.ones((T, 1), np.float32)
    y = mlp.moe(x, ids, w, gate, up, down)
    sel = lambda p: (p[0][2], p[1][2], p[2][2])
    h = mlp.linear_gated(x, sel(gate), sel(up))
    # the dense path takes bf16 input; feed the float64 H directly through the down weights
    wd, s2d = nvfp4.dequant_unscaled(down[0][2], down[1][2]), float(down[2][2])
    assert np.allclose(y, s2d * (h @ wd.T), rtol=1e-12, atol=1e-14)


def test_moe_zero_weights_give_zero():
    x, ids, w, gate, up, down = _moe_inputs(7, 4, 8, 32, 32, 923)
    y = mlp.moe(x, ids, np.zeros_like(w), gate, up, down)
    assert np.all(y == 0)


def test_moe_identical_experts_independent_of_ids():
    T, k, E, H, I = 6, 3, 5, 32, 32
    x, ids, w, gate, up, down = _moe_inputs(T, k, E, H, I, 924)
    same = lambda p: (np.repeat(p[0][:1], E, 0), np.repeat(p[1][:1], E, 0), np.repeat(p[2][:1], E, 0))
    gate, up, down = same(gate), same(up), same(down)
    w = w / w.sum(axis=1, keepdims=True)
    y1 = mlp.moe(x, ids, w, gate, up, down)
    ids2 = (ids + 1) % E
    y2 = mlp.moe(x, ids2, w, gate, up, down)
    y0 = mlp.moe(x, np.zeros((T, 1), np.int32), np.ones((T, 1), np.float32), gate, up, down)
    assert np.allclose(y1, y2, rtol=1e-6, atol=1e-9) and np.allclose(y1, y0, rtol=1e-6, atol=1e-9)


def test_moe_token_permutation_equivariant():
    T, k, E, H, I = 9, 2, 4, 32, 32
    x, ids, w, gate, up, down = _moe_inputs(T, k, E, H, I, 925)
    p = np.random.default_rng(1).permutation(T)
    y = mlp.moe(x, ids, w, gate, up, down)
    yp = mlp.moe(x[p], ids[p], w[p], gate, up, down)
    assert np.allclose(yp, y[p], rtol=1e-12, atol=1e-14)


def test_dense_mlp_vs_brute():
    M, H = 2, 32
    x = synth.bf16_normal((M, H), 1.0, 926)
    wd = _packed(H, 32, 0.5, 929)
    wg, wu = _packed(32, H, 0.5, 927), _packed(32, H, 0.5, 928)
    y = mlp.dense_mlp(x, wg, wu, wd)
    g = brute.linear(x.tolist(), wg[0].tolist(), wg[1].tolist(), wg[2], M, 32, H)
    u = brute.linear(x.tolist(), wu[0].tolist(), wu[1].tolist(), wu[2], M, 32, H)
    h = [[brute.silu(g[m][i]) * u[m][i] for i in range(32)] for m in range(M)]
    yb = [[sum(h[m][i] * brute.weight(wd[0], wd[1], wd[2], n, i) for i in range(32)) for n in range(H)]
          for m in range(M)]
    assert np.allclose(y, np.array(yb), rtol=1e-12, atol=1e-14)
