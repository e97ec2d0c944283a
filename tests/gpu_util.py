"""Helpers for the GPU parity tests: moving seeded inputs to the device, and the
parity bar for bf16 outputs (max|gpu - ref| <= 1e-2 * max|ref|, cosine >= 0.9999)."""
import numpy as np
import torch

import nvfp4_moe_expert_amd as nv

DEV = "cuda:0"
REL_MAX = 1e-2
COS_MIN = 0.9999


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(DEV)


def bf16_host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def tile32(codes: np.ndarray, scales: np.ndarray):
    """Row-major codes [G, N, K/2] and scales [G, N, K/16] -> the same bytes in the
    tiled layout of include/nvfp4.h (blocks of 32 rows): code piece (n, 32 inputs
    j..) at ((n/32)*(K/32) + j)*512 + (n%32)*16, scale piece (n, 256 inputs c..)
    at ((n/32)*(K/256) + c)*512 + (n%32)*16. Written from that definition alone."""
    codes = np.asarray(codes, np.uint8)
    scales = np.asarray(scales, np.uint8)
    squeeze = codes.ndim == 2
    if squeeze:
        codes, scales = codes[None], scales[None]
    G, N, K2 = codes.shape
    K = 2 * K2
    c = codes.reshape(G, N // 32, 32, K // 32, 16).transpose(0, 1, 3, 2, 4).reshape(G, N, K2)
    s = scales.reshape(G, N // 32, 32, K // 256, 16).transpose(0, 1, 3, 2, 4).reshape(G, N, K // 16)
    c, s = np.ascontiguousarray(c), np.ascontiguousarray(s)
    return (c[0], s[0]) if squeeze else (c, s)


def weight_dev(packed, layout: int = nv.LAYOUT_ROWS) -> nv.NVFP4Weight:
    """Oracle-packed (codes, scales, scale_2) -> device NVFP4Weight (grouped or single),
    its bytes placed in `layout` on the host."""
    codes, scales, s2 = packed
    if layout == nv.LAYOUT_TILED32:
        codes, scales = tile32(codes, scales)
    s2 = np.atleast_1d(np.asarray(s2, np.float32))
    return nv.NVFP4Weight(torch.from_numpy(np.ascontiguousarray(codes)).to(DEV),
                          torch.from_numpy(np.ascontiguousarray(scales)).to(DEV),
                          torch.from_numpy(s2).to(DEV), layout)


def assert_close(gpu: np.ndarray, ref: np.ndarray, what: str = ""):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU output"
    if ref.size == 0:
        return
    scale = np.max(np.abs(ref))
    err = np.max(np.abs(gpu - ref))
    if scale == 0:
        assert err == 0, f"{what}: reference is zero, max|gpu| = {err}"
        return
    cos = float(np.dot(gpu.ravel(), ref.ravel()) / (np.linalg.norm(gpu) * np.linalg.norm(ref)))
    assert err <= REL_MAX * scale, f"{what}: max|diff| {err:.3e} > {REL_MAX} * max|ref| {scale:.3e}"
    assert cos >= COS_MIN, f"{what}: cosine {cos:.7f} < {COS_MIN}"


def note(msg: str):
    print(f"[gpu] {msg}", flush=True)
