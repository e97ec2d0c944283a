"""The steps either side of the routed experts: the BF16 router with top-k
selection before them, the shared-expert BF16 MLP after them, and the whole MoE
block (routed + shared).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Passages (TensorFold issue #308, section "What the branch does"): the routed
experts take bf16 activations; the shared expert is a plain BF16 MLP; the dense
MLP has separate gate and up projections. The model card "GLM-5.3-Flash-NVFP4-W4A4-Experts" (section
"Quantization boundary") lists routers and shared experts among the parts that
stay BF16.

Readings (the pages give no router arithmetic; the real router's scoring is out
of scope):
* logits = x . Wr^T with Wr [E, H] bf16 (out x in), exact real products summed;
* the k largest logits are selected, ties going to the lower expert index;
* the routing weights are the softmax over the k selected logits;
* shared expert: y_s = (SiLU(x . Wsg^T) * (x . Wsu^T)) . Wsd^T with bf16 weights;
* MoE block: y = routed MLP (``mlp.moe``) + shared expert, both float64;
* BF16 routed experts (the MTP layer's draft experts kept in BF16, the
  alternative to packing them that TensorFold issue #308 asks about, "What the
  branch does"): ``moe_bf16`` is ``mlp.moe`` with bf16 weights and no tensor
  scale.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_to_f32
from .mlp import moe, silu

F64 = np.float64


def _bf(bits) -> np.ndarray:
    return bf16_to_f32(bits).astype(F64)


def router_logits(x_bits, wr_bits) -> np.ndarray:
    """[T, E] float64: logits[t, e] = sum_h x[t, h] * Wr[e, h]."""
    return _bf(x_bits) @ _bf(wr_bits).T


def topk_softmax(logits: np.ndarray, k: int):
    """Per row: the k largest values (ties to the lower index), in decreasing
    order, and the softmax over them. Returns (ids int32 [T, k], weights float64 [T, k])."""
    T, E = logits.shape
    ids = np.zeros((T, k), np.int64)
    for t in range(T):
        # decreasing value; among equal values the lower index first
        order = sorted(range(E), key=lambda e: (-logits[t, e], e))
        ids[t] = order[:k]
    sel = np.take_along_axis(logits, ids, axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    return ids.astype(np.int32), z / z.sum(axis=1, keepdims=True)


def router(x_bits, wr_bits, k: int):
    """(ids int32 [T, k], weights float64 [T, k], logits float64 [T, E])."""
    lg = router_logits(x_bits, wr_bits)
    ids, w = topk_softmax(lg, k)
    return ids, w, lg


def shared_mlp(x_bits, wg_bits, wu_bits, wd_bits) -> np.ndarray:
    """BF16 shared expert, float64: (SiLU(x.Wg^T) * (x.Wu^T)) . Wd^T, intermediate not rounded."""
    x = _bf(x_bits)
    h = silu(x @ _bf(wg_bits).T) * (x @ _bf(wu_bits).T)
    return h @ _bf(wd_bits).T


def moe_block(x_bits, wr_bits, k: int, gate, up, down, wsg_bits, wsu_bits, wsd_bits):
    """y = routed experts (routing from ``router``) + shared expert; also returns the
    routing (ids, weights, logits) for inspection."""
    ids, w, lg = router(x_bits, wr_bits, k)
    y = moe(x_bits, ids, w.astype(np.float32), gate, up, down) + shared_mlp(x_bits, wsg_bits, wsu_bits, wsd_bits)
    return y, ids, w, lg


def moe_bf16(x_bits, ids, weights, wg_bits, wu_bits, wd_bits, expert_begin: int = 0):
    """Routed expert MLP on BF16 expert weights (gate, up [E, I, H]; down [E, H, I]),
    float64, with the routing rules of ``mlp.moe``: for each local slot (t, j) of
    expert e, h = SiLU(x_t . Wg_e^T) * (x_t . Wu_e^T), y_t += w[t, j] * h . Wd_e^T."""
    x = _bf(x_bits)
    ids = np.asarray(ids, dtype=np.int64)
    w = np.asarray(weights, dtype=np.float32).astype(F64)
    T, k = ids.shape
    E = wg_bits.shape[0]
    y = np.zeros((T, x.shape[1]), F64)
    slots = np.zeros((T, k, x.shape[1]), F64)
    for e in range(E):
        tt, jj = np.nonzero(ids == e + expert_begin)
        if tt.size == 0:
            continue
        xe = x[tt]
        h = silu(xe @ _bf(wg_bits[e]).T) * (xe @ _bf(wu_bits[e]).T)
        slots[tt, jj] = h @ _bf(wd_bits[e]).T
    for j in range(k):
        y += w[:, j:j + 1] * slots[:, j]
    return y
