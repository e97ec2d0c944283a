"""NVFP4 pack (BF16 -> codes, block scales, tensor scale) and dequantization.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Stored layout (TensorFold issue #308, section "The checkpoint"): a weight
[N, K] (out x in) is kept as
  codes   [N, K/2]  uint8, element 2j in the low nibble of byte j, 2j+1 in the high;
  scales  [N, K/16] uint8, e4m3fn bits, one per 16 consecutive inputs of a row;
  scale_2 float32,  one per tensor (weight_scale_2).
The nibble order is a reading (the pages do not print it).

The pack follows ModelOpt's NVFP4 recipe, which the same issue (section "What
the branch does") applies at load time to the MTP layer's BF16 experts "a
projection at a time". The recipe as read here, every step in float32 with
correctly rounded division and no fused multiply-add:
  1. amax    = max |w| over the tensor;
  2. scale_2 = amax / 2688           (2688 = 6 * 448, e2m1 max times e4m3 max);
  3. per block of 16 along K: v = (block_amax / 6) / scale_2; the block's scale
     byte is e4m3(v), nearest-even, saturating;
  4. s_eff = e4m3_value(byte) * scale_2; each element's code is
     e2m1(w / s_eff), nearest-even, clamped at 6, sign bit of the quotient;
  5. two codes per byte, even k in the low nibble.
Readings for the degenerate cases: a tensor that is all zero gets scale_2 = 0,
scale bytes 0 and codes 0; a block whose s_eff is 0 gets codes 0.

Static activation quantization (the W4A4 form of the model card
"GLM-5.3-Flash-NVFP4-W4A4-Experts", section "Quantization boundary": NVFP4
weights with calibrated activation scales; TensorFold issue #308 notes that an
input_scale is stored beside each weight). Reading: an activation row is
quantized by steps 3-5 above with the calibrated input_scale in the place of
scale_2; nothing is computed from the activations' own amax. A block whose
amax exceeds 6 * 448 * input_scale saturates: its scale byte is 0x7E and its
codes clamp at 6.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_to_f32, e2m1_decode, e2m1_encode, e4m3_decode, e4m3_encode

GROUP = 16
F32 = np.float32


def _quantize_blocks(w: np.ndarray, gscale):
    """Steps 3-5 of the recipe for float32 values w [N, K] against the global scale
    gscale (scale_2, or an activation's input_scale): (codes [N, K/2], scale bytes [N, K/16])."""
    N, K = w.shape
    gscale = F32(gscale)
    if gscale == 0:
        return np.zeros((N, K // 2), np.uint8), np.zeros((N, K // GROUP), np.uint8)
    blocks = w.reshape(N, K // GROUP, GROUP)
    bamax = np.max(np.abs(blocks), axis=2)               # float32, exact
    with np.errstate(over="ignore"):
        v = (bamax / F32(6.0)) / gscale                  # two correctly rounded fp32 divisions
    sbyte = e4m3_encode(v)
    s_eff = e4m3_decode(sbyte).astype(F32) * gscale      # one fp32 rounding
    with np.errstate(divide="ignore", invalid="ignore"):
        q = blocks / s_eff[:, :, None]                    # fp32 division
    code = e2m1_encode(np.where(s_eff[:, :, None] == 0, F32(0.0), q))
    code = np.where(s_eff[:, :, None] == 0, np.uint8(0), code).reshape(N, K)
    codes = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return codes, sbyte.astype(np.uint8)


def pack(w_bits: np.ndarray):
    """One tensor: bf16 bits [N, K] -> (codes uint8 [N,K/2], scales uint8 [N,K/16], scale_2 float32)."""
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    N, K = w_bits.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 16")
    w = bf16_to_f32(w_bits)                               # exact
    amax = F32(np.max(np.abs(w))) if w.size else F32(0)
    scale_2 = F32(amax / F32(2688.0))
    codes, sbyte = _quantize_blocks(w, scale_2)
    return codes, sbyte, scale_2


def quantize_act(x_bits: np.ndarray, input_scale):
    """Static NVFP4 activation quantization: bf16 bits [M, K] and a calibrated fp32
    input_scale -> (codes uint8 [M, K/2], scale bytes uint8 [M, K/16]). The value
    represented is e2m1(code) * e4m3(byte) * input_scale."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    if x_bits.shape[-1] % GROUP:
        raise ValueError("K must be a multiple of 16")
    return _quantize_blocks(bf16_to_f32(x_bits), input_scale)


def pack_batch(w_bits: np.ndarray):
    """Independent pack of each tensor of a batch [G, N, K] (one scale_2 per tensor)."""
    outs = [pack(w_bits[g]) for g in range(w_bits.shape[0])]
    return (np.stack([o[0] for o in outs]), np.stack([o[1] for o in outs]),
            np.array([o[2] for o in outs], dtype=F32))


def unpack_codes(codes: np.ndarray) -> np.ndarray:
    """codes [..., K/2] -> 4-bit codes [..., K], even k from the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    out = np.empty(c.shape[:-1] + (c.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = c & 0xF
    out[..., 1::2] = c >> 4
    return out


# Value of every code and every scale byte, from the closed forms (decoded once).
_E2M1_VALUE = e2m1_decode(np.arange(16))
_E4M3_VALUE = e4m3_decode(np.arange(256))


def dequant_unscaled(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """e2m1(code) * e4m3(scale) per element, float64 [..., K]. The product of a
    1-bit-mantissa and a 3-bit-mantissa value has at most 6 significant bits and
    lies in [2^-10, 2688], so it is exact in bf16 and in float32."""
    vals = _E2M1_VALUE[unpack_codes(codes)]
    sc = np.repeat(_E4M3_VALUE[np.asarray(scales, np.uint8)], GROUP, axis=-1)
    return vals * sc


def dequant(codes, scales, scale_2):
    """(unscaled, scaled): unscaled as float32 (exact), scaled = fp32(unscaled * scale_2)."""
    u = dequant_unscaled(codes, scales).astype(F32)
    return u, (u * F32(scale_2)).astype(F32)
