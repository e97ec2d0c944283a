"""Seeded synthetic inputs for the NVFP4 routed-expert MLP.

This module only draws random inputs: bf16 activations and weights, router
outputs (expert ids and routing weights), and, for full-size GPU runs, the same
kinds of tensors drawn directly on the device. It holds none of the method's
arithmetic (no quantization, no dequantization, no GEMM, no permutation). Both
the CPU oracle and the HIP path consume what it returns.

Every draw is keyed by a tuple of integers (config seed, stream id, expert,
projection, ...). Each key gets its own independent numpy stream from
``SeedSequence``, so any tensor can be regenerated alone: a test that needs
three experts out of 288 draws only those three.

bf16 values are produced by rounding float32 draws with torch's CPU
``float32 -> bfloat16`` cast (round to nearest even), and are handed around as
``uint16`` bit patterns because numpy has no bfloat16 dtype.

The workloads follow the pages' shapes: ModelOpt NVFP4 experts of
GLM-5.3-Flash (288 routed experts per MoE layer, top-8 routing; the TensorFold
issue #308 "GLM-5.3-Flash on CUDA: read nvidia/GLM-5.3-Flash-NVFP4 (ModelOpt
NVFP4) as stored, W4A16", section "The checkpoint", and the model card
"GLM-5.3-Flash-NVFP4-W4A4-Experts", section "Quantization boundary").
"""
from __future__ import annotations

import numpy as np
import torch

# Stream ids: the second element of every key, so that streams never collide.
S_X = 1          # activations
S_W = 2          # dense / single-linear weights
S_GATE = 3       # expert gate projections
S_UP = 4         # expert up projections
S_DOWN = 5       # expert down projections
S_ROUTE = 6      # router logits / Zipf scores
S_PERM = 7       # Zipf rank permutation
S_RW = 8         # routing weights drawn directly (tests)
S_MISC = 9


def rng(*key: int) -> np.random.Generator:
    """An independent numpy generator for one integer key."""
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (torch's CPU cast, nearest even) -> uint16 bits."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_normal(shape, sigma: float, *key: int) -> np.ndarray:
    """bf16 bits of N(0, sigma^2) draws: float32 standard normal times sigma."""
    z = rng(*key).standard_normal(size=shape, dtype=np.float32)
    return f32_to_bf16_bits(z * np.float32(sigma))


def bf16_integers(shape, lo: int, hi: int, *key: int) -> np.ndarray:
    """bf16 bits of integers drawn uniformly from [lo, hi] (exact in bf16 for |v| <= 256)."""
    z = rng(*key).integers(lo, hi + 1, size=shape).astype(np.float32)
    return f32_to_bf16_bits(z)


def expert_weights(n_experts: int, n: int, k: int, sigma: float, seed: int, stream: int,
                   experts=None) -> np.ndarray:
    """bf16 bits [len(experts), n, k]; expert e is drawn from key (seed, stream, e)."""
    idx = range(n_experts) if experts is None else experts
    return np.stack([bf16_normal((n, k), sigma, seed, stream, int(e)) for e in idx])


def topk_softmax_routing(T: int, E: int, k: int, *key: int):
    """Router stand-in: logits ~ N(0,1) [T,E]; pick the k largest (ties -> lower index);
    weights = softmax over the k selected logits. Returns (ids int32 [T,k], w float32 [T,k])."""
    logits = rng(*key).standard_normal(size=(T, E))
    return _select(logits, k)


def zipf_routing(T: int, E: int, k: int, s: float, *key: int):
    """Skewed router stand-in: each expert gets a Zipf rank through a seeded permutation;
    score[t,e] = -s*ln(rank_e) + Gumbel(0,1); top-k by score. Gumbel-top-k samples k
    distinct experts without replacement with probability proportional to rank^-s.
    Weights = softmax over the selected scores."""
    g = rng(*key)
    rank = g.permutation(E) + 1
    gumbel = g.gumbel(size=(T, E))
    score = -s * np.log(rank)[None, :] + gumbel
    return _select(score, k)


def _select(score: np.ndarray, k: int):
    order = np.argsort(-score, axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(score, order, axis=1)
    sel = sel - sel.max(axis=1, keepdims=True)
    w = np.exp(sel)
    w = w / w.sum(axis=1, keepdims=True)
    return order.astype(np.int32), w.astype(np.float32)


# ---------------------------------------------------------------- device draws
def torch_bf16_normal(shape, sigma: float, seed: int, device) -> torch.Tensor:
    """N(0, sigma^2) drawn with torch's generator on `device`, rounded to bf16.
    Used for full-size inputs that would take minutes to draw on the host; the
    CPU oracle receives copies of whatever slices it checks."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    z = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    return (z * sigma).to(torch.bfloat16)
