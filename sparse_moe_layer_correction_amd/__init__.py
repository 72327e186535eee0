"""MI355X-native LatentMoE layer forward.

A thin Python binding over the C ABI of ``libmoe_mi355x.so`` (declared in
``include/moe_api.h``). Every step of the layer runs in the library's HIP
kernels; this module only checks tensor shapes and types, allocates outputs
and workspaces with torch (device memory and streams are all torch is used
for) and passes raw pointers. There is no fallback: if the library is missing
or no GPU is present, the calls raise.

The layer ("Nemotron 3 Ultra 架构 QA", CH5 Q5.1-Q5.8; the Nemotron-3 Ultra
architecture walkthrough, section "LatentMoE 层"): sigmoid router over the
uncompressed input with a bias-adjusted top-K choice and renormalised gates
scaled by routed_scaling, an H->L latent projection, K non-gated relu^2
experts L->I->L, a gate-weighted sum, the L->H projection, and a shared relu^2
expert H->Is->H on the uncompressed input, added in parallel.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Dict, Optional

__all__ = [
    "MoEError", "MoEDims", "load_library", "library_path", "EXPORTS", "route", "permute", "forward",
    "workspace_bytes", "route_workspace_bytes", "permute_workspace_bytes", "workspace_layout",
    "LatentMoE", "PhaseEvents", "forward_profiled", "PHASES", "forward_noalloc", "NOALLOC_SCRATCH_BYTES",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libmoe_mi355x.so"

# Every symbol include/moe_api.h declares.
EXPORTS = (
    "moe_route_workspace_bytes", "moe_route", "moe_permute_workspace_bytes", "moe_permute",
    "moe_workspace_bytes", "moe_workspace_layout", "moe_forward", "moe_forward_profiled", "moe_status_string",
    "moe_abi_version", "moe_quantize_mxfp8", "moe_forward_mx", "moe_forward_mx_profiled",
    "moe_rmsnorm", "moe_block_workspace_bytes", "moe_block_forward", "moe_bias_update", "moe_quantize_mxfp4",
    "moe_forward_noalloc",
)

# MOE_NOALLOC_SCRATCH_BYTES of include/moe_api.h
NOALLOC_SCRATCH_BYTES = 128 << 20

# enum moe_phase of include/moe_api.h
PHASES = ("router_split", "router_gemm", "topk", "permute", "fc1_shared_up", "expert_up", "expert_down",
          "combine", "fc2_shared_down")


class MoEError(RuntimeError):
    pass


class _Dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("L", ctypes.c_int32), ("E", ctypes.c_int32),
                ("I", ctypes.c_int32), ("K", ctypes.c_int32), ("Is", ctypes.c_int32),
                ("routed_scaling", ctypes.c_float), ("n_group", ctypes.c_int32), ("topk_group", ctypes.c_int32)]


class _Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w_router", "corr_bias", "w_fc1", "w_up", "w_down", "w_fc2",
                                              "w_sh_up", "w_sh_down")]


class _ExpertsMx(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w_up", "w_up_scale", "w_down", "w_down_scale")] + \
        [("format", ctypes.c_int32)]


MX_FORMATS = {"mxfp8": 0, "mxfp4": 1}


_LAYOUT_FIELDS = ("idx", "gate", "gap", "offsets", "row_token", "slot_row", "z", "h", "y", "y_lat", "hs", "total")


class _Layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in _LAYOUT_FIELDS]


@dataclass(frozen=True)
class MoEDims:
    T: int
    H: int
    L: int
    E: int
    I: int
    K: int
    Is: int
    routed_scaling: float = 5.0
    n_group: int = 1          # group-limited routing (1 / 1: plain top-K over all experts)
    topk_group: int = 1

    def c(self) -> _Dims:
        return _Dims(self.T, self.H, self.L, self.E, self.I, self.K, self.Is, self.routed_scaling,
                     self.n_group, self.topk_group)


_lib = None


def library_path() -> str:
    return os.environ.get("MOE_MI355X_LIB", os.path.join(_PKG, LIB_NAME))


def load_library(path: Optional[str] = None):
    """Load the HIP library (built by ``python -m sparse_moe_layer_correction_amd.build``)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or library_path()
    if not os.path.exists(p):
        raise MoEError(f"{p} not found: build it with `python -m sparse_moe_layer_correction_amd.build`")
    lib = ctypes.CDLL(p)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    dims_p = ctypes.POINTER(_Dims)
    sig = {
        "moe_route_workspace_bytes": (sz, [dims_p]),
        "moe_permute_workspace_bytes": (sz, [dims_p]),
        "moe_workspace_bytes": (sz, [dims_p]),
        "moe_workspace_layout": (i32, [dims_p, ctypes.POINTER(_Layout)]),
        "moe_route": (i32, [dims_p, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "moe_permute": (i32, [dims_p, vp, vp, ctypes.c_int32, vp, vp, vp, vp, vp, sz, vp]),
        "moe_forward": (i32, [dims_p, ctypes.POINTER(_Weights), vp, vp, vp, sz, vp]),
        "moe_forward_profiled": (i32, [dims_p, ctypes.POINTER(_Weights), vp, vp, vp, sz, vp,
                                       ctypes.POINTER(ctypes.c_void_p), i32]),
        "moe_status_string": (ctypes.c_char_p, [i32]),
        "moe_abi_version": (i32, []),
        "moe_quantize_mxfp8": (i32, [vp, ctypes.c_int64, ctypes.c_int32, vp, vp, vp]),
        "moe_quantize_mxfp4": (i32, [vp, ctypes.c_int64, ctypes.c_int32, vp, vp, vp]),
        "moe_forward_mx": (i32, [dims_p, ctypes.POINTER(_Weights), ctypes.POINTER(_ExpertsMx), vp, vp, vp, sz, vp]),
        "moe_forward_mx_profiled": (i32, [dims_p, ctypes.POINTER(_Weights), ctypes.POINTER(_ExpertsMx), vp, vp, vp,
                                          sz, vp, ctypes.POINTER(ctypes.c_void_p), i32]),
        "moe_rmsnorm": (i32, [vp, vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, vp, vp]),
        "moe_block_workspace_bytes": (sz, [dims_p]),
        "moe_block_forward": (i32, [dims_p, ctypes.POINTER(_Weights), ctypes.POINTER(_ExpertsMx), vp, ctypes.c_float,
                                    vp, vp, vp, sz, vp]),
        "moe_bias_update": (i32, [vp, ctypes.c_int32, ctypes.c_float, vp, vp]),
        "moe_forward_noalloc": (i32, [dims_p, ctypes.POINTER(_Weights), vp, vp, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def _check(rc: int):
    if rc != 0:
        raise MoEError(f"moe call failed ({rc}): {load_library().moe_status_string(rc).decode()}")


# ----------------------------------------------------------------------------
# tensor plumbing
# ----------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t, name, dtype, shape, device):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_cuda or (device is not None and t.device != device):
        raise ValueError(f"{name} must be on the GPU device {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(stream) -> int:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _workspace(nbytes: int, device, ws=None):
    torch = _torch()
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise MoEError(f"workspace too small: need {nbytes} bytes")
        return ws
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def route_workspace_bytes(dims: MoEDims) -> int:
    d = dims.c()
    return load_library().moe_route_workspace_bytes(ctypes.byref(d))


def permute_workspace_bytes(dims: MoEDims) -> int:
    d = dims.c()
    return load_library().moe_permute_workspace_bytes(ctypes.byref(d))


def workspace_bytes(dims: MoEDims) -> int:
    d = dims.c()
    return load_library().moe_workspace_bytes(ctypes.byref(d))


def workspace_layout(dims: MoEDims) -> Dict[str, int]:
    d = dims.c()
    lay = _Layout()
    _check(load_library().moe_workspace_layout(ctypes.byref(d), ctypes.byref(lay)))
    return {n: getattr(lay, n) for n in _LAYOUT_FIELDS}


# ----------------------------------------------------------------------------
# the three calls of the C ABI
# ----------------------------------------------------------------------------

def route(x, w_router, corr_bias, K: int, routed_scaling: float = 5.0, *, with_gap: bool = True,
          ws=None, stream=None, n_group: int = 1, topk_group: int = 1):
    """Router: returns (topk_idx [T,K] int32, topk_gate [T,K] fp32, gap [T] fp32 or None)."""
    torch = _torch()
    T, H = x.shape
    E = w_router.shape[0]
    dev = x.device
    _need(x, "x", torch.bfloat16, (T, H), dev)
    _need(w_router, "w_router", torch.float32, (E, H), dev)
    _need(corr_bias, "corr_bias", torch.float32, (E,), dev)
    dims = MoEDims(T, H, 64, E, 64, K, 64, routed_scaling, n_group, topk_group)
    d = dims.c()
    lib = load_library()
    idx = torch.empty(T, K, dtype=torch.int32, device=dev)
    gate = torch.empty(T, K, dtype=torch.float32, device=dev)
    gap = torch.empty(T, dtype=torch.float32, device=dev) if with_gap else None
    nbytes = lib.moe_route_workspace_bytes(ctypes.byref(d))
    if nbytes == 0:
        _check(lib.moe_route(ctypes.byref(d), None, None, None, None, None, None, None, 0, None))
    w = _workspace(nbytes, dev, ws)
    _check(lib.moe_route(ctypes.byref(d), _ptr(x), _ptr(w_router), _ptr(corr_bias), _ptr(idx), _ptr(gate),
                         _ptr(gap), _ptr(w), nbytes, _stream(stream)))
    return idx, gate, gap


def permute(topk_idx, E: int, src=None, *, ws=None, stream=None):
    """Group the T*K slots by expert (tokens ascending within an expert).

    Returns (expert_offsets [E+1], row_token [T*K], slot_row [T,K], dst [T*K,C] or None)."""
    torch = _torch()
    T, K = topk_idx.shape
    dev = topk_idx.device
    _need(topk_idx, "topk_idx", torch.int32, (T, K), dev)
    C = 0
    if src is not None:
        C = src.shape[1]
        _need(src, "src", torch.bfloat16, (T, C), dev)
    dims = MoEDims(T, 64, 64, E, 64, K, 64)
    d = dims.c()
    lib = load_library()
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    row_token = torch.empty(T * K, dtype=torch.int32, device=dev)
    slot_row = torch.empty(T, K, dtype=torch.int32, device=dev)
    dst = torch.empty(T * K, C, dtype=torch.bfloat16, device=dev) if src is not None else None
    nbytes = lib.moe_permute_workspace_bytes(ctypes.byref(d))
    if nbytes == 0:
        _check(lib.moe_permute(ctypes.byref(d), None, None, 0, None, None, None, None, None, 0, None))
    w = _workspace(nbytes, dev, ws)
    _check(lib.moe_permute(ctypes.byref(d), _ptr(topk_idx), _ptr(src), C, _ptr(dst), _ptr(offsets),
                           _ptr(row_token), _ptr(slot_row), _ptr(w), nbytes, _stream(stream)))
    return offsets, row_token, slot_row, dst


_WEIGHT_SPECS = ("w_router", "corr_bias", "w_fc1", "w_up", "w_down", "w_fc2", "w_sh_up", "w_sh_down")


def _weight_struct(dims: MoEDims, w: Dict, dev, experts: bool = True):
    """experts=False: the bf16 expert weights are not needed (MX experts given apart)."""
    torch = _torch()
    H, L, E, I, Is = dims.H, dims.L, dims.E, dims.I, dims.Is
    shapes = {"w_router": ((E, H), torch.float32), "corr_bias": ((E,), torch.float32),
              "w_fc1": ((L, H), torch.bfloat16), "w_up": ((E, I, L), torch.bfloat16),
              "w_down": ((E, L, I), torch.bfloat16), "w_fc2": ((H, L), torch.bfloat16),
              "w_sh_up": ((Is, H), torch.bfloat16), "w_sh_down": ((H, Is), torch.bfloat16)}
    names = [n for n in _WEIGHT_SPECS if experts or n not in ("w_up", "w_down")]
    for n in names:
        shp, dt = shapes[n]
        _need(w[n], n, dt, shp, dev)
    return _Weights(*[_ptr(w[n]) if n in names else None for n in _WEIGHT_SPECS])


# ----------------------------------------------------------------------------
# MX (MXFP8 / MXFP4) expert weights
# ----------------------------------------------------------------------------

def quantize_mxfp8(w, *, stream=None):
    """moe_quantize_mxfp8: bf16 [..., C] (C a multiple of 32) -> (codes uint8 [..., C],
    scales uint8 [..., C/32])."""
    torch = _torch()
    if not isinstance(w, torch.Tensor) or w.dtype != torch.bfloat16 or not w.is_cuda or not w.is_contiguous():
        raise TypeError("w must be a contiguous bf16 CUDA tensor")
    C = w.shape[-1]
    rows = w.numel() // C
    codes = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
    scales = torch.empty(w.shape[:-1] + (C // 32,), dtype=torch.uint8, device=w.device)
    _check(load_library().moe_quantize_mxfp8(_ptr(w), rows, C, _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


def quantize_mxfp4(w, *, stream=None):
    """moe_quantize_mxfp4: bf16 [..., C] (C a multiple of 32) -> (packed codes uint8 [..., C/2],
    scales uint8 [..., C/32])."""
    torch = _torch()
    if not isinstance(w, torch.Tensor) or w.dtype != torch.bfloat16 or not w.is_cuda or not w.is_contiguous():
        raise TypeError("w must be a contiguous bf16 CUDA tensor")
    C = w.shape[-1]
    rows = w.numel() // C
    codes = torch.empty(w.shape[:-1] + (C // 2,), dtype=torch.uint8, device=w.device)
    scales = torch.empty(w.shape[:-1] + (C // 32,), dtype=torch.uint8, device=w.device)
    _check(load_library().moe_quantize_mxfp4(_ptr(w), rows, C, _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


def quantize_experts_mx(weights: Dict, fmt: str = "mxfp8", *, stream=None) -> Dict:
    """The routed experts' weights of ``weights`` in MX format ``fmt`` ("mxfp8" or "mxfp4"):
    the keys of moe_experts_mx plus "format"."""
    q = {"mxfp8": quantize_mxfp8, "mxfp4": quantize_mxfp4}[fmt]
    up, up_s = q(weights["w_up"], stream=stream)
    down, down_s = q(weights["w_down"], stream=stream)
    return {"w_up": up, "w_up_scale": up_s, "w_down": down, "w_down_scale": down_s, "format": MX_FORMATS[fmt]}


def quantize_experts_mxfp8(weights: Dict, *, stream=None) -> Dict:
    """The routed experts' weights of ``weights`` as MXFP8 (keys of moe_experts_mx)."""
    return quantize_experts_mx(weights, "mxfp8", stream=stream)


def _mx_struct(dims: MoEDims, mx: Dict, dev):
    torch = _torch()
    E, L, I = dims.E, dims.L, dims.I
    fmt = int(mx.get("format", 0))
    per = 2 if fmt == 1 else 1                      # elements per code byte
    shapes = {"w_up": (E, I, L // per), "w_up_scale": (E, I, L // 32), "w_down": (E, L, I // per),
              "w_down_scale": (E, L, I // 32)}
    for n, shp in shapes.items():
        _need(mx[n], n, torch.uint8, shp, dev)
    return _ExpertsMx(*[_ptr(mx[n]) for n in ("w_up", "w_up_scale", "w_down", "w_down_scale")], fmt)


def dims_from_mx(x, weights: Dict, mx: Dict, K: int, routed_scaling: float = 5.0, n_group: int = 1,
                 topk_group: int = 1) -> MoEDims:
    T, H = x.shape
    E, I = mx["w_up"].shape[:2]
    L = mx["w_up_scale"].shape[2] * 32
    Is = weights["w_sh_up"].shape[0]
    return MoEDims(T, H, L, E, I, K, Is, routed_scaling, n_group, topk_group)


def forward_mx(x, weights: Dict, mx: Dict, K: int, routed_scaling: float = 5.0, *, out=None, ws=None,
               stream=None, n_group: int = 1, topk_group: int = 1):
    """moe_forward_mx: the forward with MX expert weights ``mx`` (quantize_experts_mx; T <= 64)."""
    torch = _torch()
    dims = dims_from_mx(x, weights, mx, K, routed_scaling, n_group, topk_group)
    dev = x.device
    _need(x, "x", torch.bfloat16, (dims.T, dims.H), dev)
    wstruct = _weight_struct(dims, weights, dev, experts=False)
    mstruct = _mx_struct(dims, mx, dev)
    d = dims.c()
    lib = load_library()
    if out is None:
        out = torch.empty(dims.T, dims.H, dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, (dims.T, dims.H), dev)
    nbytes = lib.moe_workspace_bytes(ctypes.byref(d))
    if nbytes == 0:
        _check(lib.moe_forward_mx(ctypes.byref(d), ctypes.byref(wstruct), ctypes.byref(mstruct), None, None, None, 0,
                                  None))
    w = _workspace(nbytes, dev, ws)
    _check(lib.moe_forward_mx(ctypes.byref(d), ctypes.byref(wstruct), ctypes.byref(mstruct), _ptr(x), _ptr(out),
                              _ptr(w), w.numel() * w.element_size(), _stream(stream)))
    return out


def forward_mx_profiled(x, weights: Dict, mx: Dict, K: int, routed_scaling: float, events: "PhaseEvents", *, out,
                        ws, stream=None):
    """moe_forward_mx_profiled: forward_mx with an event recorded before each phase."""
    torch = _torch()
    dims = dims_from_mx(x, weights, mx, K, routed_scaling)
    dev = x.device
    _need(x, "x", torch.bfloat16, (dims.T, dims.H), dev)
    _need(out, "out", torch.bfloat16, (dims.T, dims.H), dev)
    wstruct = _weight_struct(dims, weights, dev, experts=False)
    mstruct = _mx_struct(dims, mx, dev)
    d = dims.c()
    _check(load_library().moe_forward_mx_profiled(ctypes.byref(d), ctypes.byref(wstruct), ctypes.byref(mstruct),
                                                  _ptr(x), _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
                                                  _stream(stream), events.events, events.n))
    return out


def dims_from(x, weights: Dict, K: int, routed_scaling: float = 5.0, n_group: int = 1,
              topk_group: int = 1) -> MoEDims:
    T, H = x.shape
    E, I, L = weights["w_up"].shape
    Is = weights["w_sh_up"].shape[0]
    return MoEDims(T, H, L, E, I, K, Is, routed_scaling, n_group, topk_group)


def forward(x, weights: Dict, K: int, routed_scaling: float = 5.0, *, out=None, ws=None, stream=None,
            n_group: int = 1, topk_group: int = 1):
    """Whole layer forward; returns out [T,H] bf16. ``ws`` (uint8, >= workspace_bytes) keeps
    the intermediates at the offsets of ``workspace_layout``."""
    torch = _torch()
    dims = dims_from(x, weights, K, routed_scaling, n_group, topk_group)
    dev = x.device
    _need(x, "x", torch.bfloat16, (dims.T, dims.H), dev)
    wstruct = _weight_struct(dims, weights, dev)
    d = dims.c()
    lib = load_library()
    if out is None:
        out = torch.empty(dims.T, dims.H, dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, (dims.T, dims.H), dev)
    nbytes = lib.moe_workspace_bytes(ctypes.byref(d))
    if nbytes == 0:
        _check(lib.moe_forward(ctypes.byref(d), ctypes.byref(wstruct), None, None, None, 0, None))
    w = _workspace(nbytes, dev, ws)
    _check(lib.moe_forward(ctypes.byref(d), ctypes.byref(wstruct), _ptr(x), _ptr(out), _ptr(w),
                           w.numel() * w.element_size(), _stream(stream)))
    return out


def forward_noalloc(x, weights: Dict, K: int, routed_scaling: float = 5.0, *, out=None, stream=None,
                    n_group: int = 1, topk_group: int = 1):
    """moe_forward_noalloc: the forward with the library's static device scratch as
    its workspace (no allocation by the library; ``out`` is allocated here only
    when not given). Raises for batches whose workspace exceeds that scratch."""
    torch = _torch()
    dims = dims_from(x, weights, K, routed_scaling, n_group, topk_group)
    dev = x.device
    _need(x, "x", torch.bfloat16, (dims.T, dims.H), dev)
    wstruct = _weight_struct(dims, weights, dev)
    if out is None:
        out = torch.empty(dims.T, dims.H, dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, (dims.T, dims.H), dev)
    d = dims.c()
    _check(load_library().moe_forward_noalloc(ctypes.byref(d), ctypes.byref(wstruct), _ptr(x), _ptr(out),
                                              _stream(stream)))
    return out


# ----------------------------------------------------------------------------
# the layer's neighbours: pre-norm, residual (the block), bias update
# ----------------------------------------------------------------------------

RMS_EPS = 1e-5


def rmsnorm(x, gamma, eps: float = RMS_EPS, *, out=None, stream=None):
    """moe_rmsnorm: y = bf16(gamma * bf16(x * rsqrt(mean(x^2) + eps))) per row; x [T, H], gamma [H] bf16."""
    torch = _torch()
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise TypeError("x must be a [T, H] torch tensor")
    T, H = x.shape
    dev = x.device
    _need(x, "x", torch.bfloat16, (T, H), dev)
    _need(gamma, "gamma", torch.bfloat16, (H,), dev)
    if out is None:
        out = torch.empty_like(x)
    _need(out, "out", torch.bfloat16, (T, H), dev)
    _check(load_library().moe_rmsnorm(_ptr(x), _ptr(gamma), T, H, eps, _ptr(out), _stream(stream)))
    return out


def block_workspace_bytes(dims: MoEDims) -> int:
    return int(load_library().moe_block_workspace_bytes(ctypes.byref(dims.c())))


def block_forward(x, weights: Dict, gamma, K: int, routed_scaling: float = 5.0, eps: float = RMS_EPS, *, mx=None,
                  out=None, ws=None, stream=None, n_group: int = 1, topk_group: int = 1):
    """moe_block_forward: out = x + LatentMoE(RMSNorm(x)); ``mx`` optional MX experts (T <= 64).
    ``out`` may be ``x`` (in place)."""
    torch = _torch()
    if mx is None:
        dims = dims_from(x, weights, K, routed_scaling, n_group, topk_group)
    else:
        dims = dims_from_mx(x, weights, mx, K, routed_scaling, n_group, topk_group)
    dev = x.device
    _need(x, "x", torch.bfloat16, (dims.T, dims.H), dev)
    _need(gamma, "gamma", torch.bfloat16, (dims.H,), dev)
    wstruct = _weight_struct(dims, weights, dev, experts=mx is None)
    mstruct = None if mx is None else ctypes.byref(_mx_struct(dims, mx, dev))
    d = dims.c()
    lib = load_library()
    if out is None:
        out = torch.empty(dims.T, dims.H, dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, (dims.T, dims.H), dev)
    nbytes = lib.moe_block_workspace_bytes(ctypes.byref(d))
    if nbytes == 0:
        _check(lib.moe_block_forward(ctypes.byref(d), ctypes.byref(wstruct), mstruct, None, eps, None, None, None, 0,
                                     None))
    w = _workspace(nbytes, dev, ws)
    _check(lib.moe_block_forward(ctypes.byref(d), ctypes.byref(wstruct), mstruct, _ptr(gamma), eps, _ptr(x),
                                 _ptr(out), _ptr(w), w.numel() * w.element_size(), _stream(stream)))
    return out


def bias_update(offsets, corr_bias, eta: float, *, stream=None):
    """moe_bias_update: corr_bias[i] -= eta * (load_i - mean load), load from the expert offsets [E+1]."""
    torch = _torch()
    E = corr_bias.shape[0]
    dev = corr_bias.device
    _need(corr_bias, "corr_bias", torch.float32, (E,), dev)
    _need(offsets, "offsets", torch.int32, (E + 1,), dev)
    _check(load_library().moe_bias_update(_ptr(offsets), E, eta, _ptr(corr_bias), _stream(stream)))
    return corr_bias


class PhaseEvents:
    """HIP events for moe_forward_profiled, created through the HIP runtime."""

    def __init__(self, n: int = len(PHASES) + 1):
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.events = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            if self._hip.hipEventCreate(ctypes.byref(ev)) != 0:
                raise MoEError("hipEventCreate failed")
            self.events[i] = ev
        self.n = n

    def phase_ms(self):
        """Duration of each phase of the last recorded forward (after a synchronize)."""
        out = []
        for i in range(self.n - 1):
            ms = ctypes.c_float()
            if self._hip.hipEventElapsedTime(ctypes.byref(ms), self.events[i], self.events[i + 1]) != 0:
                raise MoEError("hipEventElapsedTime failed")
            out.append(ms.value)
        return dict(zip(PHASES, out))

    def __del__(self):
        try:
            for i in range(self.n):
                self._hip.hipEventDestroy(self.events[i])
        except Exception:
            pass


def forward_profiled(x, weights: Dict, K: int, routed_scaling: float, events: "PhaseEvents", *, out, ws,
                     stream=None):
    """moe_forward_profiled: the forward with an event recorded before each phase."""
    torch = _torch()
    dims = dims_from(x, weights, K, routed_scaling)
    dev = x.device
    _need(x, "x", torch.bfloat16, (dims.T, dims.H), dev)
    _need(out, "out", torch.bfloat16, (dims.T, dims.H), dev)
    wstruct = _weight_struct(dims, weights, dev)
    d = dims.c()
    _check(load_library().moe_forward_profiled(ctypes.byref(d), ctypes.byref(wstruct), _ptr(x), _ptr(out),
                                               _ptr(ws), ws.numel() * ws.element_size(), _stream(stream),
                                               events.events, events.n))
    return out


class LatentMoE:
    """The layer with its weights and a reusable workspace (no allocation per call)."""

    def __init__(self, weights: Dict, K: int, routed_scaling: float = 5.0, max_tokens: int = 1):
        self.weights = weights
        self.K = K
        self.routed_scaling = routed_scaling
        self._ws = None
        self._ws_tokens = 0
        self.reserve(max_tokens)

    def reserve(self, tokens: int):
        torch = _torch()
        w = self.weights
        E, I, L = w["w_up"].shape
        dims = MoEDims(tokens, w["w_fc1"].shape[1], L, E, I, self.K, w["w_sh_up"].shape[0], self.routed_scaling)
        if tokens > self._ws_tokens:
            self._ws = torch.empty(workspace_bytes(dims), dtype=torch.uint8, device=w["w_fc1"].device)
            self._ws_tokens = tokens

    def __call__(self, x, out=None, stream=None):
        self.reserve(x.shape[0])
        return forward(x, self.weights, self.K, self.routed_scaling, out=out, ws=self._ws, stream=stream)

    @property
    def workspace(self):
        return self._ws
