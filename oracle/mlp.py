"""Dense Fp4Linear, expert permutation and routed expert MLP.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Every contraction is float64 over exactly dequantized weights and widened bf16
inputs, so it stands for the real-number result; the GPU's bf16 outputs are
compared against it within a tolerance.

Passages:
* Dense MLP on Fp4Linear with separate gate and up projections, because each
  has its own tensor scale (TensorFold issue #308, section "What the branch
  does").
* Routed experts in one grouped NVFP4 kernel on bf16 activations (W4A16), each
  expert's weight_scale_2 applied to its product (same section).
* A prompt-shaped kernel whose sums do not change with how the prompt is
  chunked (same issue, "Questions", item 4), and batches executed
  deterministically (model card "GLM-5.3-Flash-NVFP4-W4A4-Experts", opening
  section).

Readings: scale_2 multiplies the contraction (it is a per-tensor scalar, so it
factors out of the sum); SiLU(z) = z / (1 + exp(-z)); the routing weight
multiplies each expert's down-projection output and the k products of a token
are summed; a slot whose id is outside [expert_begin, expert_begin + E)
contributes nothing; duplicate ids in one token count separately.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_to_f32, f32_to_bf16
from .nvfp4 import dequant_unscaled, quantize_act

F64 = np.float64


def _w64(w):
    """Weight tuple (codes [N,K/2], scales [N,K/16], scale_2) -> (unscaled float64 [N,K], scale_2 float64)."""
    codes, scales, s2 = w
    return dequant_unscaled(codes, scales), F64(np.float32(s2))


def linear(x_bits: np.ndarray, w) -> np.ndarray:
    """Y[m, n] = scale_2 * sum_k x[m, k] * (e2m1(code[n,k]) * e4m3(scale[n, k/16])), float64."""
    x = bf16_to_f32(x_bits).astype(F64)
    wu, s2 = _w64(w)
    return s2 * (x @ wu.T)


def silu(z):
    z = np.asarray(z, dtype=F64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def linear_gated(x_bits: np.ndarray, w_gate, w_up) -> np.ndarray:
    """H = SiLU(Y_gate) * Y_up with Y_gate, Y_up from ``linear`` (each its own scale_2)."""
    return silu(linear(x_bits, w_gate)) * linear(x_bits, w_up)


def dense_mlp(x_bits: np.ndarray, w_gate, w_up, w_down) -> np.ndarray:
    """Dense MLP on Fp4Linear: Y = s2d * (SiLU(Y_gate) * Y_up) . Wd^T, all float64
    (the intermediate is not rounded)."""
    h = linear_gated(x_bits, w_gate, w_up)
    wd, s2d = _w64(w_down)
    return s2d * (h @ wd.T)


def route(ids: np.ndarray, n_experts: int, expert_begin: int = 0):
    """Group the T*k slots by expert.

    Slot s = t*k + j holds ids[t, j]; it is local iff expert_begin <= id <
    expert_begin + n_experts. Returns
      counts  [E]   rows per local expert,
      offsets [E+1] exclusive prefix sums of counts,
      perm    [V]   the valid slots ordered by (local expert, slot)  -- stable,
      inv     [S]   position of each slot in perm, -1 for skipped slots.
    Written as the definition: for each expert in turn, its slots in slot order."""
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    local = flat - expert_begin
    valid = (local >= 0) & (local < n_experts)
    perm_parts, counts = [], np.zeros(n_experts, dtype=np.int64)
    for e in range(n_experts):
        slots = np.nonzero(valid & (local == e))[0]
        counts[e] = slots.size
        perm_parts.append(slots)
    perm = np.concatenate(perm_parts) if perm_parts else np.zeros(0, np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    inv = -np.ones(flat.size, dtype=np.int64)
    inv[perm] = np.arange(perm.size)
    return (counts.astype(np.int32), offsets.astype(np.int32), perm.astype(np.int32), inv.astype(np.int32))


def moe(x_bits, ids, weights, gate, up, down, expert_begin: int = 0, return_slots: bool = False):
    """Routed expert MLP, float64.

    x_bits [T, H] bf16 bits; ids [T, k] int; weights [T, k] float32;
    gate, up: (codes [E, I, H/2], scales [E, I, H/16], scale_2 [E]);
    down:     (codes [E, H, I/2], scales [E, H, I/16], scale_2 [E]).
    For every local slot (t, j) with expert e:
      g = s2g[e] * x_t . Wg_e^T,  u = s2u[e] * x_t . Wu_e^T,  h = SiLU(g) * u,
      d = s2d[e] * h . Wd_e^T,    y_t += weights[t, j] * d.
    Experts are dequantized one at a time."""
    x = bf16_to_f32(x_bits).astype(F64)
    ids = np.asarray(ids, dtype=np.int64)
    w = np.asarray(weights, dtype=np.float32).astype(F64)
    T, k = ids.shape
    H = x.shape[1]
    E = gate[0].shape[0]
    y = np.zeros((T, H), F64)
    slots = np.zeros((T, k, H), F64)
    for e in range(E):
        tt, jj = np.nonzero(ids == e + expert_begin)
        if tt.size == 0:
            continue
        wg, s2g = _w64((gate[0][e], gate[1][e], gate[2][e]))
        wu, s2u = _w64((up[0][e], up[1][e], up[2][e]))
        wd, s2d = _w64((down[0][e], down[1][e], down[2][e]))
        xe = x[tt]
        h = silu(s2g * (xe @ wg.T)) * (s2u * (xe @ wu.T))
        d = s2d * (h @ wd.T)
        slots[tt, jj] = d
    for j in range(k):
        y += w[:, j:j + 1] * slots[:, j]
    if return_slots:
        return y, slots
    return y


def act_fake_quant(x_bits, input_scale) -> np.ndarray:
    """bf16 activations -> the values their static NVFP4 quantization represents,
    e2m1(code) * e4m3(byte) * input_scale, float64 (exact: a 6-significant-bit
    value times a float32)."""
    codes, scales = quantize_act(x_bits, input_scale)
    return dequant_unscaled(codes, scales) * F64(np.float32(input_scale))


def moe_w4a4(x_bits, ids, weights, gate, up, down, in_scale_gu, in_scale_d, expert_begin: int = 0):
    """Routed expert MLP with W4A4 activations (the checkpoint's own FP4 x FP4 math,
    TensorFold issue #308, "What the branch does" and "Questions", item 1; model
    card "GLM-5.3-Flash-NVFP4-W4A4-Experts", "Quantization boundary").

    As ``moe``, with two activation quantizations, each against one calibrated
    scale for all experts of the layer (the card's activation-scale policy takes a
    percentile across experts per projection):
      x_t -> act_fake_quant(x_t, in_scale_gu) before gate/up;
      h   -> bf16(h) (rounded through float32, as the intermediate is stored), then
             act_fake_quant(., in_scale_d) before down.
    The contractions are float64 as in ``moe``."""
    xq = act_fake_quant(x_bits, in_scale_gu)
    ids = np.asarray(ids, dtype=np.int64)
    w = np.asarray(weights, dtype=np.float32).astype(F64)
    T, k = ids.shape
    H = xq.shape[1]
    E = gate[0].shape[0]
    y = np.zeros((T, H), F64)
    slots = np.zeros((T, k, H), F64)
    for e in range(E):
        tt, jj = np.nonzero(ids == e + expert_begin)
        if tt.size == 0:
            continue
        wg, s2g = _w64((gate[0][e], gate[1][e], gate[2][e]))
        wu, s2u = _w64((up[0][e], up[1][e], up[2][e]))
        wd, s2d = _w64((down[0][e], down[1][e], down[2][e]))
        xe = xq[tt]
        h = silu(s2g * (xe @ wg.T)) * (s2u * (xe @ wu.T))
        h_bits = f32_to_bf16(h.astype(np.float32))
        hq = act_fake_quant(h_bits, in_scale_d)
        slots[tt, jj] = s2d * (hq @ wd.T)
    for j in range(k):
        y += w[:, j:j + 1] * slots[:, j]
    return y
