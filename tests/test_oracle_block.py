"""Pins for oracle.block: brute-force logits, a library sort for the top-k
selection, hand-made ties, the softmax's closed form, the reduction of the BF16
shared expert to the pinned dense NVFP4 MLP when the bf16 weights are exactly
NVFP4 values, and the block's invariants."""
import numpy as np
import pytest

import synth
from oracle import block, brute, formats as F, mlp, nvfp4


def test_router_logits_vs_brute():
    T, E, H = 3, 5, 32
    x = synth.bf16_normal((T, H), 1.0, 960)
    wr = synth.bf16_normal((E, H), 0.5, 961)
    lg = block.router_logits(x, wr)
    for t in range(T):
        for e in range(E):
            ref = sum(brute._bf16(x[t, h]) * brute._bf16(wr[e, h]) for h in range(H))
            assert abs(lg[t, e] - ref) <= 1e-12 * max(1.0, abs(ref))


@pytest.mark.parametrize("T,E,k", [(40, 288, 8), (7, 16, 4), (5, 3, 3)])
def test_topk_matches_stable_argsort(T, E, k):
    lg = np.random.default_rng(962 + E).standard_normal((T, E))
    ids, w = block.topk_softmax(lg, k)
    ref = np.argsort(-lg, axis=1, kind="stable")[:, :k]
    assert np.array_equal(ids, ref)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    sel = np.take_along_axis(lg, ref, axis=1)
    # softmax closed form: w_i / w_j = exp(l_i - l_j)
    assert np.allclose(w[:, 1:] / w[:, :1], np.exp(sel[:, 1:] - sel[:, :1]), rtol=1e-12)


def test_topk_ties_go_to_the_lower_index():
    lg = np.array([[1.0, 3.0, 3.0, 0.5, 3.0],
                   [2.0, 2.0, 2.0, 2.0, 2.0]])
    ids, w = block.topk_softmax(lg, 2)
    assert ids.tolist() == [[1, 2], [0, 1]]
    assert np.allclose(w, 0.5)


def test_shared_mlp_reduces_to_dense_nvfp4_mlp():
    # bf16 weights that are exactly NVFP4 values with scale_2 = 1: the BF16 shared
    # expert and the pinned dense NVFP4 MLP compute the same function
    H, Is, T = 64, 32, 5
    g = np.random.default_rng(963)

    def exact_weight(n, k):
        codes4 = g.integers(0, 16, (n, k)).astype(np.uint8)
        codes = (codes4[:, 0::2] | (codes4[:, 1::2] << 4)).astype(np.uint8)
        scales = g.integers(0x28, 0x40, (n, k // 16)).astype(np.uint8)
        vals = nvfp4.dequant_unscaled(codes, scales)
        bits = F.f32_to_bf16(vals.astype(np.float32))
        assert np.array_equal(F.bf16_to_f32(bits).astype(np.float64), vals)
        return bits, (codes, scales, np.float32(1.0))

    (bg, pg), (bu, pu), (bd, pd) = exact_weight(Is, H), exact_weight(Is, H), exact_weight(H, Is)
    x = synth.bf16_normal((T, H), 1.0, 964)
    ys = block.shared_mlp(x, bg, bu, bd)
    yd = mlp.dense_mlp(x, pg, pu, pd)
    assert np.allclose(ys, yd, rtol=1e-12, atol=1e-12 * np.max(np.abs(yd)))


def test_moe_block_is_routed_plus_shared_and_permutes():
    T, E, H, I, Is, k = 6, 4, 32, 32, 32, 2
    x = synth.bf16_normal((T, H), 1.0, 965)
    wr = synth.bf16_normal((E, H), 0.3, 966)
    gate = nvfp4.pack_batch(synth.bf16_normal((E, I, H), 0.3, 967))
    up = nvfp4.pack_batch(synth.bf16_normal((E, I, H), 0.3, 968))
    down = nvfp4.pack_batch(synth.bf16_normal((E, H, I), 0.3, 969))
    sg, su, sd = (synth.bf16_normal(s, 0.3, 970 + i) for i, s in enumerate([(Is, H), (Is, H), (H, Is)]))
    y, ids, w, lg = block.moe_block(x, wr, k, gate, up, down, sg, su, sd)
    ref = mlp.moe(x, ids, w.astype(np.float32), gate, up, down) + block.shared_mlp(x, sg, su, sd)
    assert np.array_equal(y, ref)
    p = np.random.default_rng(971).permutation(T)
    yp, idp, _, _ = block.moe_block(x[p], wr, k, gate, up, down, sg, su, sd)
    assert np.array_equal(idp, ids[p])
    assert np.allclose(yp, y[p], rtol=1e-13, atol=1e-13 * np.max(np.abs(y)))


def test_moe_bf16_reduces_to_nvfp4_moe_on_exact_weights():
    # bf16 expert weights that are exactly NVFP4 values with scale_2 = 1: the BF16
    # routed MLP and the pinned NVFP4 routed MLP are the same function
    T, k, E, H, I = 7, 2, 3, 64, 32
    g = np.random.default_rng(972)

    def exact(n, kk):
        c4 = g.integers(0, 16, (E, n, kk)).astype(np.uint8)
        codes = (c4[..., 0::2] | (c4[..., 1::2] << 4)).astype(np.uint8)
        scales = g.integers(0x28, 0x40, (E, n, kk // 16)).astype(np.uint8)
        vals = nvfp4.dequant_unscaled(codes, scales)
        bits = F.f32_to_bf16(vals.astype(np.float32))
        assert np.array_equal(F.bf16_to_f32(bits).astype(np.float64), vals)
        return bits, (codes, scales, np.ones(E, np.float32))

    (bg, pg), (bu, pu), (bd, pd) = exact(I, H), exact(I, H), exact(H, I)
    x = synth.bf16_normal((T, H), 1.0, 973)
    ids, w = synth.topk_softmax_routing(T, E, k, 974)
    yb = block.moe_bf16(x, ids, w, bg, bu, bd)
    yn = mlp.moe(x, ids, w, pg, pu, pd)
    assert np.allclose(yb, yn, rtol=1e-12, atol=1e-12 * np.max(np.abs(yn)))
    # skipped ids contribute nothing
    assert not block.moe_bf16(x, ids, w, bg, bu, bd, expert_begin=E).any()
