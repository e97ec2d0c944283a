"""MI355X-native W4A16 NVFP4 routed-expert MLP.

Thin ctypes binding over ``libnvfp4.so`` (C ABI in ``include/nvfp4.h``). This
module only marshals arguments: it checks dtypes, shapes and contiguity,
passes device pointers and the current HIP stream, and allocates outputs and
workspaces with torch. Every step of the computation runs in the library's
HIP kernels; there is no fallback. If the library is missing, every call
raises.

The weight format is the ModelOpt NVFP4 one read "as stored" (TensorFold issue
#308, section "The checkpoint"): codes [G, N, K/2] uint8 (even k in the low
nibble), scales [G, N, K/16] e4m3fn bytes, scale_2 [G] float32. The same bytes
can also sit in the library's tiled layout (LAYOUT_TILED32, blocks of 32 rows,
see include/nvfp4.h); the tensors keep their shapes as byte containers then.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

__all__ = [
    "Nvfp4Error", "NVFP4Weight", "load_library", "library_path", "abi_version", "ABI_VERSION",
    "pack", "relayout", "dequant", "selftest_fp4_convert", "linear", "linear_gated", "moe_route", "moe_grouped",
    "moe_workspace_size", "pack_workspace_size", "moe_plan", "LAYOUT_ROWS", "LAYOUT_TILED32",
    "CLASS_AUTO", "CLASS_DECODE", "CLASS_PREFILL", "KERNEL_NAMES", "moe_grouped_noalloc", "NOALLOC_SCRATCH_BYTES",
]

# interface version this binding was written against (NVFP4_ABI_VERSION in include/nvfp4.h)
ABI_VERSION = 8

LAYOUT_ROWS = 0       # the checkpoint's row-major codes and scales
LAYOUT_TILED32 = 1    # blocks of 32 rows (n % 32 == 0, k % 256 == 0)

# kernel classes of the routed GEMMs (NVFP4_CLASS_* in include/nvfp4.h)
CLASS_AUTO = 0
CLASS_DECODE = 1
CLASS_PREFILL = 2
# kernels named by moe_plan (NVFP4_KERNEL_*)
KERNEL_NAMES = {0: "none", 1: "decode_ksplit", 2: "decode", 3: "decode_resident", 4: "prefill", 5: "fallback", 6: "tiny"}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libnvfp4.so")
_lib = None


class Nvfp4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = load_library().nvfp4_status_string(status).decode()
        super().__init__(f"{where}: nvfp4 status {status} ({msg})")


class _Weight(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("scale_2", ctypes.c_void_p),
                ("n", ctypes.c_int64), ("k", ctypes.c_int64), ("groups", ctypes.c_int32),
                ("layout", ctypes.c_int32)]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t
_WP = ctypes.POINTER(_Weight)

_SIGNATURES = {
    "nvfp4_abi_version": (ctypes.c_int, []),
    "nvfp4_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "nvfp4_pack_workspace_size": (_SZ, [_I32, _I64, _I64]),
    "nvfp4_pack": (ctypes.c_int, [_P, _I32, _I64, _I64, _P, _P, _P, _P, _SZ, _I32, _P]),
    "nvfp4_relayout": (ctypes.c_int, [_WP, _WP, _P]),
    "nvfp4_dequant": (ctypes.c_int, [_WP, _P, _P, _P]),
    "nvfp4_selftest_fp4_convert": (ctypes.c_int, [_P, _P]),
    "nvfp4_linear": (ctypes.c_int, [_P, _I64, _WP, _P, _P]),
    "nvfp4_linear_gated": (ctypes.c_int, [_P, _I64, _WP, _WP, _P, _P]),
    "nvfp4_moe_route_workspace_size": (_SZ, [_I64, _I32, _I32]),
    "nvfp4_moe_route": (ctypes.c_int, [_P, _I64, _I32, _I32, _I32, _P, _P, _P, _P, _SZ, _P]),
    "nvfp4_moe_workspace_size": (_SZ, [_I64, _I32, _I32, _I64, _I64]),
    "nvfp4_moe_grouped": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _I32, _I32, _WP, _WP, _WP, _P, _SZ, _P, _P]),
    "nvfp4_moe_grouped_class": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _I32, _I32, _WP, _WP, _WP, _I32, _P, _SZ,
                                               _P, _P]),
    "nvfp4_moe_plan": (ctypes.c_int, [_I64, _I32, _I32, _I64, _I64, _I32, _I32, _I32, ctypes.POINTER(_I32)]),
    "nvfp4_moe_grouped_noalloc": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _I32, _I32, _WP, _WP, _WP, _P, _P]),
    "nvfp4_moe_grouped_timed": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _I32, _I32, _WP, _WP, _WP, _P, _SZ, _P,
                                               _P, ctypes.POINTER(_P)]),
    "nvfp4_moe_grouped_w4a4": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _I32, _I32, _WP, _WP, _WP, _P, _P, _P, _SZ,
                                              _P, _P]),
    "nvfp4_quantize_act": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P, _P]),
    "nvfp4_router_workspace_size": (_SZ, [_I64, _I64, _I32]),
    "nvfp4_router_topk": (ctypes.c_int, [_P, _I64, _I64, _P, _I32, _I32, _P, _SZ, _P, _P, _P]),
    "nvfp4_bf16_mlp_workspace_size": (_SZ, [_I64, _I64, _I64]),
    "nvfp4_bf16_mlp": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P, _I64, _P, _SZ, _P, _P]),
    "nvfp4_moe_block_workspace_size": (_SZ, [_I64, _I32, _I32, _I64, _I64, _I64]),
    "nvfp4_moe_block": (ctypes.c_int, [_P, _I64, _I64, _P, _I32, _WP, _WP, _WP, _P, _P, _P, _I64, _P, _SZ, _P, _P]),
    "nvfp4_moe_grouped_bf16_workspace_size": (_SZ, [_I64, _I32, _I32, _I64, _I64]),
    "nvfp4_moe_grouped_bf16": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _I32, _I32, _P, _P, _P, _I32, _I64, _P, _SZ,
                                              _P, _P]),
}


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libnvfp4.so (built in-tree by ``python -m nvfp4_moe_expert_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with `python -m nvfp4_moe_expert_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if lib.nvfp4_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{_LIB_PATH} has ABI version {lib.nvfp4_abi_version()}, the binding expects "
                               f"{ABI_VERSION}: rebuild it")
        _lib = lib
    return _lib


def abi_version() -> int:
    return load_library().nvfp4_abi_version()


# ---------------------------------------------------------------- helpers
def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t: torch.Tensor | None) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _need(t: torch.Tensor, dtype: torch.dtype, name: str, ndim: int | None = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (W4A16: activations are bf16 rows), got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous row-major")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


def _check(status: int, where: str):
    if status != 0:
        raise Nvfp4Error(status, where)


@dataclass
class NVFP4Weight:
    """Device tensors of one NVFP4 weight or a group of them (experts)."""
    codes: torch.Tensor    # uint8 [G, N, K/2]
    scales: torch.Tensor   # uint8 [G, N, K/16]
    scale_2: torch.Tensor  # float32 [G]
    layout: int = LAYOUT_ROWS

    def __post_init__(self):
        if self.codes.dim() == 2:
            self.codes = self.codes.unsqueeze(0)
        if self.scales.dim() == 2:
            self.scales = self.scales.unsqueeze(0)
        if self.scale_2.dim() == 0:
            self.scale_2 = self.scale_2.reshape(1)
        _need(self.codes, torch.uint8, "codes", 3)
        _need(self.scales, torch.uint8, "scales", 3)
        _need(self.scale_2, torch.float32, "scale_2", 1)
        g, n, k2 = self.codes.shape
        if self.scales.shape != (g, n, k2 * 2 // 16) or self.scale_2.shape != (g,):
            raise ValueError("inconsistent NVFP4 weight shapes")
        if self.layout not in (LAYOUT_ROWS, LAYOUT_TILED32):
            raise ValueError(f"unknown layout {self.layout}")

    @property
    def groups(self) -> int:
        return self.codes.shape[0]

    @property
    def n(self) -> int:
        return self.codes.shape[1]

    @property
    def k(self) -> int:
        return self.codes.shape[2] * 2

    def _struct(self) -> _Weight:
        return _Weight(self.codes.data_ptr(), self.scales.data_ptr(), self.scale_2.data_ptr(),
                       self.n, self.k, self.groups, self.layout)

    def expert(self, e: int) -> "NVFP4Weight":
        # one tensor's bytes are one contiguous block in either layout
        return NVFP4Weight(self.codes[e:e + 1], self.scales[e:e + 1], self.scale_2[e:e + 1], self.layout)


# ---------------------------------------------------------------- entry points
def pack_workspace_size(batch: int, n: int, k: int) -> int:
    return load_library().nvfp4_pack_workspace_size(batch, n, k)


def pack(w: torch.Tensor, layout: int = LAYOUT_ROWS) -> NVFP4Weight:
    """BF16 [N, K] or [G, N, K] -> NVFP4 (one scale_2 per tensor), in `layout`."""
    lib = load_library()
    if w.dim() == 2:
        w = w.unsqueeze(0)
    _need(w, torch.bfloat16, "w", 3)
    g, n, k = w.shape
    dev = w.device
    codes = torch.empty((g, n, k // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((g, n, k // 16), dtype=torch.uint8, device=dev)
    s2 = torch.empty((g,), dtype=torch.float32, device=dev)
    wsb = max(lib.nvfp4_pack_workspace_size(g, n, k), 16)
    ws = torch.empty((wsb,), dtype=torch.uint8, device=dev)
    _check(lib.nvfp4_pack(_ptr(w), g, n, k, _ptr(codes), _ptr(scales), _ptr(s2), _ptr(ws), wsb, layout,
                          _stream()), "nvfp4_pack")
    return NVFP4Weight(codes, scales, s2, layout)


def relayout(w: NVFP4Weight, layout: int) -> NVFP4Weight:
    """The same weight with its codes and scales in `layout` (new tensors; scale_2 shared)."""
    lib = load_library()
    out = NVFP4Weight(torch.empty_like(w.codes), torch.empty_like(w.scales), w.scale_2, layout)
    src, dst = w._struct(), out._struct()
    _check(lib.nvfp4_relayout(ctypes.byref(src), ctypes.byref(dst), _stream()), "nvfp4_relayout")
    return out


def dequant(w: NVFP4Weight, unscaled: bool = True, scaled: bool = True):
    """(bf16 [G,N,K] code*scale, fp32 [G,N,K] code*scale*scale_2); either may be None."""
    lib = load_library()
    dev = w.codes.device
    u = torch.empty((w.groups, w.n, w.k), dtype=torch.bfloat16, device=dev) if unscaled else None
    s = torch.empty((w.groups, w.n, w.k), dtype=torch.float32, device=dev) if scaled else None
    ws = w._struct()
    _check(lib.nvfp4_dequant(ctypes.byref(ws), _ptr(u), _ptr(s), _stream()), "nvfp4_dequant")
    return u, s


def linear(x: torch.Tensor, w: NVFP4Weight, out: torch.Tensor | None = None) -> torch.Tensor:
    """y[m, n] = bf16(scale_2 * x . W^T)."""
    lib = load_library()
    _need(x, torch.bfloat16, "x", 2)
    if out is None:
        out = torch.empty((x.shape[0], w.n), dtype=torch.bfloat16, device=x.device)
    _need(out, torch.bfloat16, "out", 2)
    if x.shape[1] != w.k or out.shape != (x.shape[0], w.n):
        raise ValueError("shape mismatch in linear")
    ws = w._struct()
    _check(lib.nvfp4_linear(_ptr(x), x.shape[0], ctypes.byref(ws), _ptr(out), _stream()), "nvfp4_linear")
    return out


def linear_gated(x: torch.Tensor, w_gate: NVFP4Weight, w_up: NVFP4Weight,
                 out: torch.Tensor | None = None) -> torch.Tensor:
    """h[m, n] = bf16(SiLU(gate) * up), gate and up each with their own scale_2."""
    lib = load_library()
    _need(x, torch.bfloat16, "x", 2)
    if out is None:
        out = torch.empty((x.shape[0], w_gate.n), dtype=torch.bfloat16, device=x.device)
    _need(out, torch.bfloat16, "out", 2)
    if x.shape[1] != w_gate.k or out.shape != (x.shape[0], w_gate.n):
        raise ValueError("shape mismatch in linear_gated")
    g, u = w_gate._struct(), w_up._struct()
    _check(lib.nvfp4_linear_gated(_ptr(x), x.shape[0], ctypes.byref(g), ctypes.byref(u), _ptr(out), _stream()),
           "nvfp4_linear_gated")
    return out


def selftest_fp4_convert(device="cuda") -> int:
    """Inputs (of all 2^32 fp32 patterns, NaNs skipped, with their negations) whose
    device fp4 convert differs from the e2m1 rounding the pack uses; 0 expected."""
    lib = load_library()
    out = torch.empty((1,), dtype=torch.int64, device=device)
    _check(lib.nvfp4_selftest_fp4_convert(_ptr(out), _stream()), "nvfp4_selftest_fp4_convert")
    return int(out.item())


def moe_route(topk_ids: torch.Tensor, n_experts: int, expert_begin: int = 0, scratch: bool = True):
    """(offsets [E+1], perm [T*k] (valid prefix), inv [T*k]) - the stable permutation by expert.

    scratch=False passes no workspace, so one workgroup routes every batch size."""
    lib = load_library()
    _need(topk_ids, torch.int32, "topk_ids", 2)
    T, k = topk_ids.shape
    dev = topk_ids.device
    offsets = torch.empty((n_experts + 1,), dtype=torch.int32, device=dev)
    perm = torch.empty((max(T * k, 1),), dtype=torch.int32, device=dev)
    inv = torch.empty((max(T * k, 1),), dtype=torch.int32, device=dev)
    nbytes = lib.nvfp4_moe_route_workspace_size(T, k, n_experts) if scratch else 0
    ws = torch.empty((nbytes,), dtype=torch.uint8, device=dev) if nbytes else None
    _check(lib.nvfp4_moe_route(_ptr(topk_ids), T, k, n_experts, expert_begin, _ptr(offsets), _ptr(perm),
                               _ptr(inv), _ptr(ws), nbytes, _stream()), "nvfp4_moe_route")
    return offsets, perm[: T * k], inv[: T * k]


def moe_workspace_size(T: int, k: int, n_experts: int, H: int, I: int) -> int:
    return load_library().nvfp4_moe_workspace_size(T, k, n_experts, H, I)


def moe_plan(T: int, k: int, n_experts: int, H: int, I: int, gate_layout: int = LAYOUT_ROWS,
             down_layout: int = LAYOUT_ROWS, kernel_class: int = CLASS_AUTO) -> dict:
    """The kernels a routed call of these shapes runs (nvfp4_moe_plan; host only)."""
    lib = load_library()
    plan = (_I32 * 5)()
    _check(lib.nvfp4_moe_plan(T, k, n_experts, H, I, gate_layout, down_layout, kernel_class, plan), "nvfp4_moe_plan")
    return {"tile_rows": plan[0], "gate_up": KERNEL_NAMES[plan[1]], "down": KERNEL_NAMES[plan[2]],
            "down_width": plan[3], "fp16": bool(plan[4])}


def moe_grouped(x: torch.Tensor, topk_ids: torch.Tensor, topk_w: torch.Tensor, gate: NVFP4Weight,
                up: NVFP4Weight, down: NVFP4Weight, expert_begin: int = 0, workspace: torch.Tensor | None = None,
                out: torch.Tensor | None = None, events=None, input_scales=None,
                kernel_class: int | None = None) -> torch.Tensor:
    """Routed expert MLP of one MoE layer: y[T, H] bf16.

    events: optional sequence of 5 torch.cuda.Event; the library records them on the
    current stream before the first kernel and after the route, gate/up, down and
    combine stages.
    input_scales: None (W4A16), or a float32 device tensor [2] holding the
    calibrated activation scales (gate/up input, down input) for W4A4
    (nvfp4_moe_grouped_w4a4; not combined with events).
    kernel_class: None (nvfp4_moe_grouped), or CLASS_AUTO / CLASS_DECODE /
    CLASS_PREFILL to pin the class (nvfp4_moe_grouped_class; W4A16 only, no events)."""
    lib = load_library()
    if kernel_class is not None and (input_scales is not None or events is not None):
        raise ValueError("kernel_class is taken by the W4A16 entry point without events")
    if input_scales is not None:
        _need(input_scales, torch.float32, "input_scales", 1)
        if input_scales.numel() != 2:
            raise ValueError("input_scales must hold 2 floats (gate/up input, down input)")
        if events is not None:
            raise ValueError("events are not recorded by the W4A4 entry point")
    _need(x, torch.bfloat16, "x", 2)
    _need(topk_ids, torch.int32, "topk_ids", 2)
    _need(topk_w, torch.float32, "topk_w", 2)
    T, H = x.shape
    k = topk_ids.shape[1]
    if topk_ids.shape != (T, k) or topk_w.shape != (T, k):
        raise ValueError("topk_ids / topk_w must be [T, k]")
    E, I = gate.groups, gate.n
    need = lib.nvfp4_moe_workspace_size(T, k, E, H, I)
    if workspace is None:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=x.device)
    _need(workspace, torch.uint8, "workspace", 1)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    _need(out, torch.bfloat16, "out", 2)
    g, u, d = gate._struct(), up._struct(), down._struct()
    args = (_ptr(x), T, H, _ptr(topk_ids), _ptr(topk_w), k, expert_begin, ctypes.byref(g), ctypes.byref(u),
            ctypes.byref(d), _ptr(workspace), workspace.numel(), _ptr(out), _stream())
    if input_scales is not None:
        st = lib.nvfp4_moe_grouped_w4a4(*args[:10], _ptr(input_scales), _ptr(input_scales[1:]), *args[10:])
        _check(st, "nvfp4_moe_grouped_w4a4")
        return out
    if kernel_class is not None:
        _check(lib.nvfp4_moe_grouped_class(*args[:10], kernel_class, *args[10:]), "nvfp4_moe_grouped_class")
        return out
    if events is None:
        st = lib.nvfp4_moe_grouped(*args)
    else:
        if len(events) != 5:
            raise ValueError("events must hold 5 torch.cuda.Event")
        for ev in events:          # make sure each event object exists on the device
            if ev.cuda_event == 0:
                ev.record()
        arr = (_P * 5)(*[ctypes.c_void_p(ev.cuda_event) for ev in events])
        st = lib.nvfp4_moe_grouped_timed(*args, arr)
    _check(st, "nvfp4_moe_grouped")
    return out


# fixed scratch of nvfp4_moe_grouped_noalloc (NVFP4_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20


def moe_grouped_noalloc(x: torch.Tensor, topk_ids: torch.Tensor, topk_w: torch.Tensor, gate: NVFP4Weight,
                        up: NVFP4Weight, down: NVFP4Weight, out: torch.Tensor, expert_begin: int = 0) -> torch.Tensor:
    """The routed expert MLP without a workspace (nvfp4_moe_grouped_noalloc): the
    library's fixed per-GPU scratch serves the call, so nothing is allocated;
    the caller passes the output y [T, H] bf16."""
    lib = load_library()
    _need(x, torch.bfloat16, "x", 2)
    _need(topk_ids, torch.int32, "topk_ids", 2)
    _need(topk_w, torch.float32, "topk_w", 2)
    _need(out, torch.bfloat16, "out", 2)
    T, H = x.shape
    k = topk_ids.shape[1]
    if topk_ids.shape != (T, k) or topk_w.shape != (T, k) or out.shape != (T, H):
        raise ValueError("topk_ids / topk_w must be [T, k] and out [T, H]")
    g, u, d = gate._struct(), up._struct(), down._struct()
    _check(lib.nvfp4_moe_grouped_noalloc(_ptr(x), T, H, _ptr(topk_ids), _ptr(topk_w), k, expert_begin, ctypes.byref(g),
                                         ctypes.byref(u), ctypes.byref(d), _ptr(out), _stream()),
           "nvfp4_moe_grouped_noalloc")
    return out


def quantize_act(x: torch.Tensor, input_scale: torch.Tensor):
    """Static NVFP4 activation quantization (W4A4): bf16 x [rows, k] and a float32
    device tensor holding the calibrated input_scale -> (codes uint8 [rows, k/2],
    scales uint8 [rows, k/16])."""
    lib = load_library()
    _need(x, torch.bfloat16, "x", 2)
    _need(input_scale, torch.float32, "input_scale", 1)
    rows, k = x.shape
    codes = torch.empty((rows, k // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((rows, k // 16), dtype=torch.uint8, device=x.device)
    st = lib.nvfp4_quantize_act(_ptr(x), rows, k, _ptr(input_scale), _ptr(codes), _ptr(scales), _stream())
    _check(st, "nvfp4_quantize_act")
    return codes, scales


# ---------------------------------------------------------------- BF16 steps either side
def router_topk(x: torch.Tensor, w_router: torch.Tensor, k: int, workspace: torch.Tensor | None = None):
    """Router logits x . w_router^T (fp32), top-k (ties to the lower index) and the
    softmax over the selected: (ids int32 [T, k], weights float32 [T, k])."""
    lib = load_library()
    _need(x, torch.bfloat16, "x", 2)
    _need(w_router, torch.bfloat16, "w_router", 2)
    T, H = x.shape
    E = w_router.shape[0]
    if w_router.shape[1] != H:
        raise ValueError("w_router must be [E, H]")
    if workspace is None:
        workspace = torch.empty((max(lib.nvfp4_router_workspace_size(T, H, E), 256),), dtype=torch.uint8,
                                device=x.device)
    ids = torch.empty((T, k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    _check(lib.nvfp4_router_topk(_ptr(x), T, H, _ptr(w_router), E, k, _ptr(workspace), workspace.numel(), _ptr(ids),
                                 _ptr(w), _stream()), "nvfp4_router_topk")
    return ids, w


def bf16_mlp(x: torch.Tensor, w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor,
             workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Shared-expert BF16 MLP: fp32 [M, H] = (SiLU(x.Wg^T) * (x.Wu^T)) . Wd^T."""
    lib = load_library()
    for t, n in ((x, "x"), (w_gate, "w_gate"), (w_up, "w_up"), (w_down, "w_down")):
        _need(t, torch.bfloat16, n, 2)
    M, H = x.shape
    Is = w_gate.shape[0]
    if w_gate.shape != (Is, H) or w_up.shape != (Is, H) or w_down.shape != (H, Is):
        raise ValueError("shared expert shapes: gate, up [Is, H]; down [H, Is]")
    if workspace is None:
        workspace = torch.empty((max(lib.nvfp4_bf16_mlp_workspace_size(M, H, Is), 256),), dtype=torch.uint8,
                                device=x.device)
    y = torch.empty((M, H), dtype=torch.float32, device=x.device)
    _check(lib.nvfp4_bf16_mlp(_ptr(x), M, H, _ptr(w_gate), _ptr(w_up), _ptr(w_down), Is, _ptr(workspace),
                              workspace.numel(), _ptr(y), _stream()), "nvfp4_bf16_mlp")
    return y


def moe_block(x: torch.Tensor, w_router: torch.Tensor, k: int, gate: NVFP4Weight, up: NVFP4Weight,
              down: NVFP4Weight, shared_gate: torch.Tensor, shared_up: torch.Tensor, shared_down: torch.Tensor,
              workspace: torch.Tensor | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """One MoE block: router + routed NVFP4 experts + shared BF16 expert -> y [T, H] bf16."""
    lib = load_library()
    _need(x, torch.bfloat16, "x", 2)
    for t, n in ((w_router, "w_router"), (shared_gate, "shared_gate"), (shared_up, "shared_up"),
                 (shared_down, "shared_down")):
        _need(t, torch.bfloat16, n, 2)
    T, H = x.shape
    Is = shared_gate.shape[0]
    E, I = gate.groups, gate.n
    if workspace is None:
        workspace = torch.empty((max(lib.nvfp4_moe_block_workspace_size(T, k, E, H, I, Is), 256),),
                                dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    g, u, d = gate._struct(), up._struct(), down._struct()
    _check(lib.nvfp4_moe_block(_ptr(x), T, H, _ptr(w_router), k, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d),
                               _ptr(shared_gate), _ptr(shared_up), _ptr(shared_down), Is, _ptr(workspace),
                               workspace.numel(), _ptr(out), _stream()), "nvfp4_moe_block")
    return out


def moe_block_workspace_size(T: int, k: int, n_experts: int, H: int, I: int, Is: int) -> int:
    return load_library().nvfp4_moe_block_workspace_size(T, k, n_experts, H, I, Is)


def moe_grouped_bf16(x: torch.Tensor, topk_ids: torch.Tensor, topk_w: torch.Tensor, w_gate: torch.Tensor,
                     w_up: torch.Tensor, w_down: torch.Tensor, expert_begin: int = 0,
                     workspace: torch.Tensor | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """Routed expert MLP on BF16 expert weights (gate, up [E, I, H]; down [E, H, I]): y [T, H] bf16."""
    lib = load_library()
    _need(x, torch.bfloat16, "x", 2)
    _need(topk_ids, torch.int32, "topk_ids", 2)
    _need(topk_w, torch.float32, "topk_w", 2)
    for t, n in ((w_gate, "w_gate"), (w_up, "w_up"), (w_down, "w_down")):
        _need(t, torch.bfloat16, n, 3)
    T, H = x.shape
    k = topk_ids.shape[1]
    E, I = w_gate.shape[0], w_gate.shape[1]
    if w_gate.shape != (E, I, H) or w_up.shape != (E, I, H) or w_down.shape != (E, H, I):
        raise ValueError("expert weights: gate, up [E, I, H]; down [E, H, I]")
    if workspace is None:
        workspace = torch.empty((max(lib.nvfp4_moe_grouped_bf16_workspace_size(T, k, E, H, I), 256),),
                                dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    _check(lib.nvfp4_moe_grouped_bf16(_ptr(x), T, H, _ptr(topk_ids), _ptr(topk_w), k, expert_begin, _ptr(w_gate),
                                      _ptr(w_up), _ptr(w_down), E, I, _ptr(workspace), workspace.numel(), _ptr(out),
                                      _stream()), "nvfp4_moe_grouped_bf16")
    return out


def moe_grouped_bf16_workspace_size(T: int, k: int, n_experts: int, H: int, I: int) -> int:
    return load_library().nvfp4_moe_grouped_bf16_workspace_size(T, k, n_experts, H, I)
