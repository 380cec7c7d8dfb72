"""Beam Mixture-of-Experts layer for MI355X (gfx950): Python binding of libbeam_moe.so.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  Tensors passed here must already live on the GPU (torch is used for
device memory and streams); the binding checks dtypes and shapes, hands raw
pointers to the C ABI declared in include/beam_moe.h, and raises on any nonzero
status.  There is no CPU path: if the library is missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libbeam_moe.so")

BEAM_OK, BEAM_ERR_INVALID_ARG, BEAM_ERR_UNSUPPORTED, BEAM_ERR_WORKSPACE, BEAM_ERR_HIP = range(5)
BEAM_DTYPE_F32, BEAM_DTYPE_BF16, BEAM_DTYPE_FP8_E4M3, BEAM_DTYPE_MXFP4 = range(4)
BEAM_FP8_SCALES_FP32, BEAM_FP8_SCALES_POW2 = range(2)

C_FUNCTIONS = ("beam_moe_status_string", "beam_moe_abi_version", "beam_moe_workspace_size",
               "beam_moe_workspace_map", "beam_moe_route", "beam_moe_forward",
               "beam_moe_sublayer_forward", "beam_moe_time_kernel", "beam_dense_workspace_size",
               "beam_dense_forward", "beam_dense_sublayer_forward", "beam_moe_forward_noalloc")
BEAM_KERNEL_NONE, BEAM_KERNEL_ROUTER_LOGITS, BEAM_KERNEL_GATE_UP, BEAM_KERNEL_DOWN, BEAM_KERNEL_COMBINE = range(5)


class beam_moe_config(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("n_groups", ctypes.c_int32),
                ("topk_groups", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("routed_scale", ctypes.c_float), ("act_dtype", ctypes.c_int32),
                ("weight_dtype", ctypes.c_int32), ("fp8_block", ctypes.c_int32),
                ("norm_eps", ctypes.c_float), ("fp8_scale_kind", ctypes.c_int32)]


ABI_VERSION = 5          # BEAM_MOE_ABI_VERSION of the structures below


class beam_moe_ws_map(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("logits", "expert_count", "expert_off", "row_of_pair",
                                               "pair_of_row", "hidden", "expert_out", "scores", "xhat",
                                               "x_q", "x_q_scale", "h_q", "h_q_scale", "total")]


class BeamMoEError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


def make_config(hidden=5120, inter=2560, n_experts=256, n_groups=8, topk_groups=4, topk=8,
                routed_scale=2.5, act_dtype=BEAM_DTYPE_BF16, weight_dtype=BEAM_DTYPE_BF16,
                fp8_block=128, norm_eps=1e-6, fp8_scale_kind=BEAM_FP8_SCALES_FP32) -> beam_moe_config:
    """Layer configuration; the defaults are Beam's (hidden 5120, 256 experts in 8 groups
    of 32, top-4 groups, top-8 experts, intermediate 2560, scale 2.5).  fp8_scale_kind:
    BEAM_FP8_SCALES_POW2 only when every FP8 block scale is a power of two."""
    return beam_moe_config(hidden, inter, n_experts, n_groups, topk_groups, topk, routed_scale,
                           act_dtype, weight_dtype, fp8_block, norm_eps, fp8_scale_kind)


_lib = None


def lib() -> ctypes.CDLL:
    """Load libbeam_moe.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m sparse_mixture_experts_group_amd.build` (no fallback path exists)")
    L = ctypes.CDLL(LIB_PATH)
    L.beam_moe_abi_version.restype = ctypes.c_int
    if L.beam_moe_abi_version() != ABI_VERSION:
        raise ImportError(f"{LIB_PATH} has ABI {L.beam_moe_abi_version()}, this binding expects {ABI_VERSION}: "
                          "rebuild it with `python -m sparse_mixture_experts_group_amd.build`")
    vp, cfgp = ctypes.c_void_p, ctypes.POINTER(beam_moe_config)
    i64, sz = ctypes.c_int64, ctypes.c_size_t
    L.beam_moe_status_string.restype = ctypes.c_char_p
    L.beam_moe_status_string.argtypes = [ctypes.c_int]
    L.beam_moe_abi_version.restype = ctypes.c_int
    L.beam_moe_workspace_size.restype = sz
    L.beam_moe_workspace_size.argtypes = [cfgp, i64]
    L.beam_moe_workspace_map.restype = ctypes.c_int
    L.beam_moe_workspace_map.argtypes = [cfgp, i64, ctypes.POINTER(beam_moe_ws_map)]
    L.beam_moe_route.restype = ctypes.c_int
    L.beam_moe_route.argtypes = [cfgp, i64, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.beam_moe_forward.restype = ctypes.c_int
    L.beam_moe_forward.argtypes = [cfgp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.beam_moe_sublayer_forward.restype = ctypes.c_int
    L.beam_moe_sublayer_forward.argtypes = [cfgp, i64, vp, vp, vp, ctypes.c_int32, vp, vp, vp, vp, vp,
                                            vp, vp, vp, vp, vp, vp, sz, vp]
    L.beam_moe_time_kernel.restype = ctypes.c_int
    L.beam_moe_time_kernel.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_void_p), ctypes.c_int]
    L.beam_dense_workspace_size.restype = sz
    L.beam_dense_workspace_size.argtypes = [cfgp, i64]
    L.beam_dense_forward.restype = ctypes.c_int
    L.beam_dense_forward.argtypes = [cfgp, i64, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.beam_moe_forward_noalloc.restype = ctypes.c_int
    L.beam_moe_forward_noalloc.argtypes = [cfgp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.beam_dense_sublayer_forward.restype = ctypes.c_int
    L.beam_dense_sublayer_forward.argtypes = [cfgp, i64, vp, vp, vp, ctypes.c_int32, vp, vp, vp, vp, vp, vp, sz,
                                              vp]
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().beam_moe_status_string(int(status)).decode()


def abi_version() -> int:
    return int(lib().beam_moe_abi_version())


def beam_moe_workspace_size(cfg: beam_moe_config, T: int) -> int:
    return int(lib().beam_moe_workspace_size(ctypes.byref(cfg), int(T)))


def beam_moe_workspace_map(cfg: beam_moe_config, T: int) -> dict:
    m = beam_moe_ws_map()
    st = lib().beam_moe_workspace_map(ctypes.byref(cfg), int(T), ctypes.byref(m))
    if st != BEAM_OK:
        raise BeamMoEError(st, "beam_moe_workspace_map")
    return {n: int(getattr(m, n)) for n, _ in beam_moe_ws_map._fields_}


# ---------------------------------------------------------------------------
# tensor marshalling
# ---------------------------------------------------------------------------
def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(st: int, where: str):
    if st != BEAM_OK:
        raise BeamMoEError(st, where)


def alloc_workspace(cfg: beam_moe_config, T: int, device="cuda"):
    """Device workspace (uint8 tensor) sized by beam_moe_workspace_size."""
    import torch
    n = beam_moe_workspace_size(cfg, T)
    if n == 0 and T > 0:
        raise BeamMoEError(BEAM_ERR_INVALID_ARG, "beam_moe_workspace_size")
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def beam_moe_route(cfg, x, w_router, logit_bias=None, ids=None, weights=None, ws=None, stream=None,
                   select_bias=None):
    """Router: returns (ids [T,K] int32, weights [T,K] float32) on the GPU."""
    import torch
    T = x.shape[0]
    K = cfg.topk
    ids = torch.empty((T, K), dtype=torch.int32, device=x.device) if ids is None else ids
    weights = torch.empty((T, K), dtype=torch.float32, device=x.device) if weights is None else weights
    ws = alloc_workspace(cfg, T, x.device) if ws is None else ws
    st = lib().beam_moe_route(ctypes.byref(cfg), T, _ptr(x), _ptr(w_router), _ptr(logit_bias), _ptr(select_bias),
                              _ptr(ids), _ptr(weights), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "beam_moe_route")
    return ids, weights


def beam_moe_forward(cfg, x, w_router, w13, w2, logit_bias=None, w13_scale=None, w2_scale=None, y=None,
                     ids=None, weights=None, ws=None, stream=None, select_bias=None):
    """One MoE layer: returns y [T,H] (same dtype as x) on the GPU."""
    import torch
    T = x.shape[0]
    y = torch.empty_like(x) if y is None else y
    ws = alloc_workspace(cfg, T, x.device) if ws is None else ws
    st = lib().beam_moe_forward(ctypes.byref(cfg), T, _ptr(x), _ptr(w_router), _ptr(logit_bias),
                                _ptr(select_bias), _ptr(w13), _ptr(w13_scale), _ptr(w2), _ptr(w2_scale), _ptr(y), _ptr(ids), _ptr(weights),
                                _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "beam_moe_forward")
    return y


NOALLOC_SCRATCH_BYTES = 64 << 20       # BEAM_MOE_NOALLOC_SCRATCH_BYTES


def beam_moe_forward_noalloc(cfg, x, w_router, w13, w2, logit_bias=None, w13_scale=None, w2_scale=None, y=None,
                             ids=None, weights=None, stream=None, select_bias=None):
    """beam_moe_forward on the library's static per-device scratch array (no workspace;
    the library allocates nothing).  y must be given by callers that cannot allocate."""
    import torch
    T = x.shape[0]
    y = torch.empty_like(x) if y is None else y
    st = lib().beam_moe_forward_noalloc(ctypes.byref(cfg), T, _ptr(x), _ptr(w_router), _ptr(logit_bias),
                                        _ptr(select_bias), _ptr(w13), _ptr(w13_scale), _ptr(w2), _ptr(w2_scale),
                                        _ptr(y), _ptr(ids), _ptr(weights), _stream(stream))
    _check(st, "beam_moe_forward_noalloc")
    return y


class KernelTimer:
    """Brackets the next `n` launches of one library kernel with torch CUDA events
    (recorded by the library on the launch stream).  Use as a context manager; after
    synchronising, `times_ms()` gives each bracketed launch's duration."""

    def __init__(self, kernel: int, n: int):
        import torch
        self.kernel, self.n = kernel, n
        self.events = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)]
        for e in self.events:          # torch creates the HIP event on its first record
            e.record()
        torch.cuda.synchronize()
        self._arr = (ctypes.c_void_p * (2 * n))(*[e.cuda_event for e in self.events])

    def __enter__(self):
        _check(lib().beam_moe_time_kernel(self.kernel, self._arr, self.n), "beam_moe_time_kernel")
        return self

    def __exit__(self, *exc):
        lib().beam_moe_time_kernel(BEAM_KERNEL_NONE, None, 0)
        return False

    def times_ms(self):
        return [self.events[2 * i].elapsed_time(self.events[2 * i + 1]) for i in range(self.n)]


def beam_moe_sublayer_forward(cfg, h, step_k, w_router, w13, w2, pre_gain=None, post_gain=None,
                              logit_bias=None, w13_scale=None, w2_scale=None, moe_out=None, ids=None,
                              weights=None, ws=None, stream=None, select_bias=None):
    """pre-RMSNorm -> MoE -> post-RMSNorm -> constant-scale residual, updating h in place."""
    T = h.shape[0]
    ws = alloc_workspace(cfg, T, h.device) if ws is None else ws
    st = lib().beam_moe_sublayer_forward(ctypes.byref(cfg), T, _ptr(h), _ptr(pre_gain), _ptr(post_gain),
                                         int(step_k), _ptr(w_router), _ptr(logit_bias), _ptr(select_bias),
                                         _ptr(w13),
                                         _ptr(w13_scale), _ptr(w2), _ptr(w2_scale), _ptr(moe_out), _ptr(ids),
                                         _ptr(weights), _ptr(ws), ws.numel() * ws.element_size(),
                                         _stream(stream))
    _check(st, "beam_moe_sublayer_forward")
    return h


# ---------------------------------------------------------------------------
# dense SwiGLU MLP (the first decoder layers)
# ---------------------------------------------------------------------------
def make_dense_config(hidden=5120, inter=20480, act_dtype=BEAM_DTYPE_BF16, weight_dtype=BEAM_DTYPE_BF16,
                      fp8_block=128, norm_eps=1e-6, fp8_scale_kind=BEAM_FP8_SCALES_FP32) -> beam_moe_config:
    """Configuration of the dense MLP (only these fields are read; the router fields are
    left at their defaults).  The default width 20480 is a reading (8 x 2560), not a
    number on the pages."""
    return make_config(hidden=hidden, inter=inter, act_dtype=act_dtype, weight_dtype=weight_dtype,
                       fp8_block=fp8_block, norm_eps=norm_eps, fp8_scale_kind=fp8_scale_kind)


def beam_dense_workspace_size(cfg: beam_moe_config, T: int) -> int:
    return int(lib().beam_dense_workspace_size(ctypes.byref(cfg), int(T)))


def alloc_dense_workspace(cfg: beam_moe_config, T: int, device="cuda"):
    """Device workspace (uint8 tensor) sized by beam_dense_workspace_size."""
    import torch
    n = beam_dense_workspace_size(cfg, T)
    if n == 0 and T > 0:
        raise BeamMoEError(BEAM_ERR_INVALID_ARG, "beam_dense_workspace_size")
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def beam_dense_forward(cfg, x, w13, w2, w13_scale=None, w2_scale=None, y=None, ws=None, stream=None):
    """Dense SwiGLU MLP: returns y [T,H] (same dtype as x) on the GPU."""
    import torch
    T = x.shape[0]
    y = torch.empty_like(x) if y is None else y
    ws = alloc_dense_workspace(cfg, T, x.device) if ws is None else ws
    st = lib().beam_dense_forward(ctypes.byref(cfg), T, _ptr(x), _ptr(w13), _ptr(w13_scale), _ptr(w2),
                                  _ptr(w2_scale), _ptr(y), _ptr(ws), ws.numel() * ws.element_size(),
                                  _stream(stream))
    _check(st, "beam_dense_forward")
    return y


def beam_dense_sublayer_forward(cfg, h, step_k, w13, w2, pre_gain=None, post_gain=None, w13_scale=None,
                                w2_scale=None, mlp_out=None, ws=None, stream=None):
    """pre-RMSNorm -> dense MLP -> post-RMSNorm -> constant-scale residual, updating h in place."""
    T = h.shape[0]
    ws = alloc_dense_workspace(cfg, T, h.device) if ws is None else ws
    st = lib().beam_dense_sublayer_forward(ctypes.byref(cfg), T, _ptr(h), _ptr(pre_gain), _ptr(post_gain),
                                           int(step_k), _ptr(w13), _ptr(w13_scale), _ptr(w2), _ptr(w2_scale),
                                           _ptr(mlp_out), _ptr(ws), ws.numel() * ws.element_size(),
                                           _stream(stream))
    _check(st, "beam_dense_sublayer_forward")
    return h
