"""Float64 brute force on tiny shapes: scalar loops, no numpy linear algebra.

TEST INFRASTRUCTURE ONLY. These functions exist to pin the vectorised oracle:
they re-derive the same quantities element by element from the format's value
tables (not from ``formats``), so a transposed operand, a wrong nibble or a
wrong block index in the vectorised code shows up as a mismatch.
"""
from __future__ import annotations

import math
import struct

# OCP e2m1 magnitudes, code order 0..7 (sign is bit 3).
_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _e2m1(c: int) -> float:
    v = _E2M1[c & 7]
    return -v if c & 8 else v


def _e4m3(b: int) -> float:
    s, e, m = (b >> 7) & 1, (b >> 3) & 15, b & 7
    if e == 15 and m == 7:
        return math.nan
    v = m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
    return -v if s else v


def _bf16(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def weight(codes, scales, s2, n: int, k: int) -> float:
    """W[n, k] = e2m1(nibble) * e4m3(scale byte of block k//16) * scale_2."""
    byte = int(codes[n][k // 2])
    c = byte & 0xF if k % 2 == 0 else byte >> 4
    return _e2m1(c) * _e4m3(int(scales[n][k // 16])) * float(s2)


def linear(x_bits, codes, scales, s2, M: int, N: int, K: int):
    """Y[m][n] = sum_k x[m][k] * W[n][k], triple loop."""
    y = [[0.0] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += _bf16(x_bits[m][k]) * weight(codes, scales, s2, n, k)
            y[m][n] = acc
    return y


def silu(z: float) -> float:
    if z < -700:
        return 0.0 * z
    return z / (1.0 + math.exp(-z))


def moe(x_bits, ids, rw, gate, up, down, T: int, k: int, H: int, I: int, expert_begin: int = 0, E: int = None):
    """Routed MLP by loops: for each token and each of its k slots, run that expert's
    gate/up/SiLU/down on the token and add weight * output."""
    y = [[0.0] * H for _ in range(T)]
    for t in range(T):
        xt = [[int(v) for v in x_bits[t]]]
        for j in range(k):
            e = int(ids[t][j]) - expert_begin
            if e < 0 or (E is not None and e >= E):
                continue
            g = linear(xt, gate[0][e], gate[1][e], gate[2][e], 1, I, H)[0]
            u = linear(xt, up[0][e], up[1][e], up[2][e], 1, I, H)[0]
            h = [silu(g[i]) * u[i] for i in range(I)]
            d = [0.0] * H
            for n in range(H):
                acc = 0.0
                for i in range(I):
                    acc += h[i] * weight(down[0][e], down[1][e], down[2][e], n, i)
                d[n] = acc
            for n in range(H):
                y[t][n] += float(rw[t][j]) * d[n]
    return y
